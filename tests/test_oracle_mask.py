"""Pins for the oracle's attended-key set (CPU only).

The set is described on the int8 tensor-core prefill attention page (section
"Why the attention, and why tensor cores": causal + sink/window, block
granular, window start constant over a 16-row tile) and its "Relation to open
PRs" section (window <= 0 means full causal).  The same page's figure of about
2.08 TFLOP for one 32k layer at the default 256-block window pins the size of
the set at the real shape.
"""
import numpy as np
import pytest

import oracle

PAGE = 16


def brute_force_set(t, W, S):
    """Pure-Python enumeration straight from the prose: every earlier-or-same
    key whose 16-token block is one of the first S blocks or one of the last W
    blocks up to and including the query's own block."""
    own_block = t // PAGE
    keep = []
    for j in range(t + 1):
        b = j // PAGE
        if W <= 0:
            keep.append(j)
            continue
        in_window = own_block - W < b <= own_block
        in_sink = b < S
        if in_window or in_sink:
            keep.append(j)
    return keep


def closed_form_count(t, W, S):
    """Counting argument: t+1 keys before the window opens; afterwards a
    partial own block (t%16+1), W-1 full blocks before it, and the sink blocks
    that lie left of the window."""
    nb = t // PAGE + 1
    if W <= 0 or nb <= W:
        return t + 1
    first_window_block = nb - W
    return (t % PAGE + 1) + PAGE * (W - 1) + PAGE * min(S, first_window_block)


@pytest.mark.parametrize("W,S", [(0, 0), (0, 3), (1, 0), (1, 1), (2, 1), (3, 0), (1, 2),
                                 (4, 4), (5, 9), (256, 1)])
def test_mask_matches_brute_force(W, S):
    n = 300
    rows = np.arange(n)
    keys = np.arange(n)
    m = oracle.attended_mask(rows, keys, W, S)
    for t in range(n):
        expect = np.zeros(n, dtype=bool)
        expect[brute_force_set(t, W, S)] = True
        assert np.array_equal(m[t], expect), (t, W, S)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 100, 1000, 4099])
@pytest.mark.parametrize("W,S", [(0, 0), (2, 1), (3, 0), (1, 2), (8, 3), (256, 1)])
def test_counts_closed_form(n, W, S):
    got = oracle.mask_counts(n, W, S)
    expect = np.array([closed_form_count(t, W, S) for t in range(n)])
    assert np.array_equal(got, expect)


def test_window_at_least_sequence_is_causal():
    n = 777
    nblk = (n + PAGE - 1) // PAGE
    for W in (nblk, nblk + 5):
        assert np.array_equal(oracle.mask_counts(n, W, 2), np.arange(1, n + 1))
    # window off ignores the sink count
    assert np.array_equal(oracle.mask_counts(n, 0, 7), np.arange(1, n + 1))
    assert np.array_equal(oracle.mask_counts(n, -3, 7), np.arange(1, n + 1))


def test_window_start_constant_over_tile():
    """The pages: n_blk_q = (t+16)/16 is the same for the 16 rows of a tile."""
    for W in (1, 3, 256):
        for tile in range(0, 40):
            t = np.arange(tile * PAGE, tile * PAGE + PAGE)
            rsb = oracle.window_start_block(t, W)
            assert len(set(rsb.tolist())) == 1


# Sum of |A(t)| per workload, from the counting argument above.
CONFIG_SUMS = {
    "tiny": (64, 0, 0, 2080),
    "4k": (4096, 256, 1, 8390656),
    "32k": (32768, 256, 1, 126074880),
    "64k": (65536, 256, 1, 260571136),
    "16k_full": (16384, 0, 0, 134225920),
}


@pytest.mark.parametrize("name", list(CONFIG_SUMS))
def test_config_sums_closed_form(name):
    n, W, S, total = CONFIG_SUMS[name]
    assert sum(closed_form_count(t, W, S) for t in range(n)) == total


def test_oracle_counts_4k_full_enumeration():
    n, W, S, total = CONFIG_SUMS["4k"]
    assert int(oracle.mask_counts(n, W, S).sum()) == total


def test_max_keys_per_row_at_default_window():
    # sink block + 255 full window blocks + the full own block
    c = oracle.mask_counts(8192, 256, 1)
    assert c.max() == 4112
    # last row before the window slides: plain causal; first row after: the
    # window drops block 0 but the sink keeps it, and only 1 key of block 256
    assert c[4095] == 4096 and c[4096] == 4097
    assert c[-1] == 4112


def test_32k_op_count_matches_pages_figure():
    """4 ops per (score, channel) pair (QK and PV multiply-adds) over 16 query
    heads at hd256: the pages quote ~2.08 TFLOP per 32k layer."""
    n, W, S, total = CONFIG_SUMS["32k"]
    ops = 4 * total * 256 * 16
    assert abs(ops / 2.08e12 - 1) < 0.01
    # the oracle's own enumeration on a sample of 32k tiles agrees with the closed form
    for tile in (0, 1, 255, 256, 257, 1000, 2047):
        rows = np.arange(tile * PAGE, tile * PAGE + PAGE)
        keys = np.arange(0, rows[-1] + 1)
        got = oracle.attended_mask(rows, keys, W, S).sum(axis=1)
        assert np.array_equal(got, [closed_form_count(t, W, S) for t in rows])
