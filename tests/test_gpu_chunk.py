"""GPU parity of chunked prefill (wpa_prefill_attn_i8_chunk, wpa_mask_counts_chunk)
through the C ABI.

A chunk is the query rows at positions q_start .. q_start+n-1 of a longer
sequence whose keys are already in the pool.  The attended set of each row is
the one the int8 tensor-core prefill attention page defines ("Why the
attention, and why tensor cores": causal + sink/window over 16-token blocks),
so the oracle is simply the whole-sequence oracle evaluated on the chunk's
rows, and splitting a prefill into chunks must give bitwise the same rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import check_parity, upload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_chunk(case, dev, q_start, n, out_dtype=torch.bfloat16, q_key="q_bf16"):
    import windowed_int8_paged_amd as wpa
    q = dev[q_key][q_start:q_start + n].contiguous()
    q_i8, q_scale = wpa.quantize_q_rows(q)
    out = wpa.prefill_attn_i8_chunk(q_start, q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                    dev["v_scale"], dev["page_table"], case.window_blocks, case.sink_blocks,
                                    case.softmax_scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def full_rows(case, q_start, chunk_out):
    """The chunk's output placed at its rows of a whole-sequence array (NaN elsewhere)."""
    full = torch.full((case.n_tokens, case.n_q_heads, 256), float("nan"), dtype=chunk_out.dtype)
    full[q_start:q_start + chunk_out.shape[0]] = chunk_out.cpu()
    return full


@pytest.mark.parametrize("q_start,n,W,S", [(0, 50, 3, 1), (32, 10, 4, 0), (160, 100, 3, 1), (304, 1, 2, 2),
                                           (64, 200, 0, 0)])
def test_mask_counts_chunk_bit_exact(q_start, n, W, S):
    import windowed_int8_paged_amd as wpa
    got = wpa.mask_counts_chunk(q_start, n, W, S).cpu().numpy()
    assert np.array_equal(got, oracle.mask_counts(q_start + n, W, S)[q_start:])


@pytest.mark.parametrize("W,S,hq,hkv", [
    (3, 1, 8, 2), (0, 0, 8, 2), (2, 4, 8, 2),
    # fewer than four query heads per KV head: a workgroup takes 2 or 4 query
    # tiles, and the chunk edges (tiles 6 and 13) fall inside those groups
    (3, 1, 4, 2), (1, 1, 3, 3), (0, 0, 2, 2), (2, 0, 6, 2),
])
def test_chunks_equal_one_call_bitwise(W, S, hq, hkv):
    case = workloads.make_case(n_tokens=300, n_q_heads=hq, n_kv_heads=hkv, window_blocks=W, sink_blocks=S,
                               seed=21, extra_pool_frac=0.25)
    dev = upload(case)
    import windowed_int8_paged_amd as wpa
    _say(f"chunks vs one call W={W} S={S} hq={hq} hkv={hkv}")
    for dt in (torch.bfloat16, torch.float32):
        q_i8, q_scale = wpa.quantize_q_rows(dev["q_bf16"])
        one = wpa.prefill_attn_i8(q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                  dev["page_table"], W, S, case.softmax_scale, out_dtype=dt)
        parts = [run_chunk(case, dev, a, b - a, dt) for a, b in ((0, 96), (96, 208), (208, 300))]
        assert torch.equal(torch.cat(parts), one)


def test_long_call_in_xcd_runs_equals_chunks_bitwise():
    """A call long enough that each XCD takes a contiguous run of tile groups
    (512 groups per KV head) against two chunks short enough to take every
    other group: the order of the groups over the chip must not change a bit."""
    import windowed_int8_paged_amd as wpa
    case = workloads.make_case(n_tokens=16384, n_q_heads=16, n_kv_heads=4, window_blocks=256, sink_blocks=1,
                               seed=41)
    dev = upload(case)
    _say("one 16384-row call (XCD runs) vs two 8192-row chunks")
    q_i8, q_scale = wpa.quantize_q_rows(dev["q_bf16"])
    one = wpa.prefill_attn_i8(q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                              dev["page_table"], case.window_blocks, case.sink_blocks, case.softmax_scale,
                              out_dtype=torch.bfloat16)
    parts = [run_chunk(case, dev, a, 8192, torch.bfloat16) for a in (0, 8192)]
    assert torch.equal(torch.cat(parts), one)


@pytest.mark.parametrize("n_total,q_start,hq,hkv,W,S,seed", [
    (500, 320, 8, 2, 4, 2, 31),     # ragged chunk at the end, windowed
    (500, 160, 4, 1, 0, 0, 32),     # full causal, chunk in the middle
    (700, 400, 16, 4, 3, 1, 33),    # GQA-4
    (600, 208, 2, 2, 1, 1, 34),     # MHA, one-block window: four tiles per workgroup, chunk inside a group
    (600, 96, 4, 2, 2, 0, 35),      # GQA-2: two tiles per workgroup
])
def test_chunk_parity(n_total, q_start, hq, hkv, W, S, seed):
    case = workloads.make_case(n_tokens=n_total, n_q_heads=hq, n_kv_heads=hkv, window_blocks=W, sink_blocks=S,
                               seed=seed, extra_pool_frac=0.3)
    dev = upload(case)
    # the chunk ends at the sequence end (ragged last tile) or on a tile edge, so
    # the oracle's tiles hold exactly the chunk's rows
    n = n_total - q_start if seed != 32 else 192
    _say(f"chunk parity n_total={n_total} q_start={q_start} n={n} hq={hq} hkv={hkv} W={W} S={S}")
    tiles = list(range(q_start // 16, (q_start + n + 15) // 16))
    out = run_chunk(case, dev, q_start, n, torch.float32)
    r = check_parity(case, full_rows(case, q_start, out), tiles=tiles, label="chunk f32")
    _say(f"  {r}")


def test_chunk_past_64k():
    """A 4096-row chunk at position 65536 over a 69632-token cache: beyond the
    pages' 64k batched-prefill limit.  One KV head, four query heads, the
    headline window (256 blocks + 1 sink); the oracle runs on sampled tiles."""
    case = workloads.make_case(n_tokens=69632, n_q_heads=4, n_kv_heads=1, window_blocks=256, sink_blocks=1,
                               seed=41)
    dev = upload(case)
    q_start, n = 65536, 4096
    _say("chunk at 65536")
    out = run_chunk(case, dev, q_start, n, torch.bfloat16)
    tiles = [q_start // 16, q_start // 16 + 97, (q_start + n) // 16 - 1]
    r = check_parity(case, full_rows(case, q_start, out), tiles=tiles, label="chunk 64k+")
    _say(f"  {r}")


def test_chunk_rows_past_133000_keys():
    """A full-causal 16-row chunk at position 134144: each row attends about
    134000 keys, every V code is +127, and query head 0 is all zero, so its
    weights are all at full scale after the first step and the int32 PV
    planes grow by 127 * 127 per key, past 2^31 after about 133000 keys
    without the kernel's range guard.  Held to the plain bars on the chunk's
    tile; the oracle takes about half a minute on it."""
    from gpu_util import oracle_rows
    import windowed_int8_paged_amd as wpa
    n_total, q_rows, hq, hkv = 134160, 16, 4, 1
    case = workloads.make_long_row_case(n_total, q_rows, hq, hkv, seed=42)
    q_start = n_total - q_rows
    _say(f"chunk rows attending {n_total} keys")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = torch.from_numpy(case.q_bf16[q_start:].view(np.int16)).cuda().view(torch.bfloat16)
    q_i8, q_scale = wpa.quantize_q_rows(q)
    out = wpa.prefill_attn_i8_chunk(q_start, q_i8, q_scale, t(case.k_pool), t(case.v_pool), t(case.k_scale),
                                    t(case.v_scale), t(case.page_table), 0, 0, case.softmax_scale,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    rows, b, a = oracle_rows(case, [q_start // 16])
    assert np.array_equal(rows, np.arange(q_start, n_total))
    mo = np.abs(b).max()
    rel = np.abs(o - b).max() / mo
    frob = np.linalg.norm(o - a) / np.linalg.norm(a)
    _say(f"  rel_mirror {rel:.3e} frob_exact {frob:.3e}")
    assert rel <= 2e-3
    assert frob <= 3e-2
