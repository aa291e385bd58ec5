"""Pins for the oracle's per-row Q quantization (CPU only).

The int8 tensor-core prefill attention page, section "Why the attention, and
why tensor cores", quantizes Q with one scale per query row.  The expected
values below are worked by hand.
"""
import numpy as np

import oracle


def row(vals):
    r = np.zeros(256, dtype=np.float32)
    r[: len(vals)] = vals
    return r


def test_hand_worked_row():
    # amax = 2 -> step 2/127, multiplier 63.5; 1.0*63.5 = 63.5 rounds half-even to 64
    codes, scale = oracle.quantize_q_rows(row([1.0, -2.0, 0.5, 0.25])[None])
    assert codes[0, :4].tolist() == [64, -127, 32, 16]
    assert np.all(codes[0, 4:] == 0)
    assert scale[0] == np.float32(2.0) / np.float32(127.0)


def test_ties_round_half_even():
    # amax = 127/8 -> multiplier exactly 8, so q*8 is exact and lands on halves
    q = row(np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 127.0], dtype=np.float32) / 8)
    codes, scale = oracle.quantize_q_rows(q[None])
    assert codes[0, :7].tolist() == [2, 4, -2, -4, 0, 2, 127]
    assert scale[0] == np.float32(0.125)


def test_zero_row():
    codes, scale = oracle.quantize_q_rows(np.zeros((3, 256), dtype=np.float32))
    assert np.all(codes == 0) and np.all(scale == 0)


def test_codes_on_grid_roundtrip_exactly():
    rng = np.random.default_rng(3)
    c = rng.integers(-127, 128, size=(50, 256)).astype(np.int8)
    c[:, 7] = 127
    q = c.astype(np.float32) / np.float32(64)     # exactly on a grid with step 1/64
    codes, scale = oracle.quantize_q_rows(q)
    assert np.array_equal(codes, c)
    assert np.all(scale == np.float32(1 / 64))


def test_random_rows_error_bound_and_range():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((500, 3, 256)).astype(np.float32)
    q[0, 0, 5] = 40.0
    codes, scale = oracle.quantize_q_rows(q)
    assert codes.dtype == np.int8 and codes.min() >= -127
    assert np.all(np.abs(codes).max(axis=-1) == 127)     # the row max maps to +-127
    err = np.abs(codes.astype(np.float64) * scale[..., None] - q)
    assert np.all(err <= scale[..., None].astype(np.float64) * (0.5 + 1e-5))
