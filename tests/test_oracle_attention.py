"""Pins for the oracle's two attention modes (CPU only).

Mode (a) is exact masked softmax attention over the dequantized pool; mode (b)
mirrors the int8 scheme of the int8 tensor-core prefill attention page
(section "Why the attention, and why tensor cores").  Each mode is checked
against things it does not share code with: torch's scaled_dot_product_attention
in float64, a pure-Python triple loop, closed forms of special cases and a
hand-worked example under tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_oracle_mask import brute_force_set

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_case(n=77, hq=4, hkv=2, W=0, S=0, seed=11, **kw):
    return workloads.make_case(n_tokens=n, n_q_heads=hq, n_kv_heads=hkv, window_blocks=W,
                               sink_blocks=S, seed=seed, **kw)


def contiguous_kv(case):
    """Logical-order K/V, dequantized, as [Hkv][N][256] float64 (layout only)."""
    n = case.n_tokens
    tok = np.arange(n)
    phys = case.page_table[tok // 16]
    slot = tok % 16
    k = case.k_pool[phys, slot].astype(np.float64) * case.k_scale[phys, slot][..., None]
    v = case.v_pool[phys, slot].astype(np.float64) * case.v_scale[phys, slot][..., None]
    return k.transpose(1, 0, 2), v.transpose(1, 0, 2)


def sdpa_reference(case, mask=None):
    G = case.n_q_heads // case.n_kv_heads
    k, v = contiguous_kv(case)
    q = torch.from_numpy(case.q_f32.astype(np.float64).transpose(1, 0, 2).copy())
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)
    if mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(
            q, kt, vt, is_causal=True, scale=case.softmax_scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(
            q, kt, vt, attn_mask=torch.from_numpy(mask), scale=case.softmax_scale)
    return o.numpy().transpose(1, 0, 2)


def prose_mask(n, W, S):
    m = np.zeros((n, n), dtype=bool)
    for t in range(n):
        m[t, brute_force_set(t, W, S)] = True
    return m


# ---------------------------------------------------------------- mode (a)

@pytest.mark.parametrize("n,hq,hkv", [(77, 4, 2), (64, 2, 1), (33, 8, 8)])
def test_exact_full_causal_matches_sdpa(n, hq, hkv):
    case = small_case(n=n, hq=hq, hkv=hkv, W=0)
    np.testing.assert_allclose(oracle.attention_exact(case), sdpa_reference(case),
                               rtol=1e-11, atol=1e-12)


def test_exact_window_covering_sequence_is_causal():
    case = small_case(n=70, W=5, S=2)          # 5 blocks >= ceil(70/16)
    np.testing.assert_allclose(oracle.attention_exact(case), sdpa_reference(case),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("W,S", [(1, 0), (1, 1), (2, 1), (3, 0), (2, 3)])
def test_exact_window_matches_sdpa_with_prose_mask(W, S):
    case = small_case(n=150, W=W, S=S)
    ref = sdpa_reference(case, prose_mask(150, W, S))
    np.testing.assert_allclose(oracle.attention_exact(case), ref, rtol=1e-11, atol=1e-12)


def test_exact_triple_loop_brute_force():
    case = small_case(n=37, hq=2, hkv=1, W=1, S=1, seed=5)
    ref = np.zeros((37, 2, 256))
    for t in range(37):
        keys = brute_force_set(t, 1, 1)
        for h in range(2):
            scores = []
            for j in keys:
                p, s = case.page_table[j // 16], j % 16
                dot = 0.0
                for d in range(256):
                    dot += float(case.q_f32[t, h, d]) * float(case.k_pool[p, s, 0, d]) \
                        * float(case.k_scale[p, s, 0])
                scores.append(dot * case.softmax_scale)
            mx = max(scores)
            w = [math.exp(x - mx) for x in scores]
            tot = sum(w)
            for wi, j in zip(w, keys):
                p, s = case.page_table[j // 16], j % 16
                ref[t, h] += (wi / tot) * case.v_pool[p, s, 0].astype(np.float64) \
                    * float(case.v_scale[p, s, 0])
    np.testing.assert_allclose(oracle.attention_exact(case), ref, rtol=1e-10, atol=1e-12)


def test_exact_row0_and_zero_query_mean():
    case = small_case(n=50, W=2, S=1)
    k, v = contiguous_kv(case)
    out = oracle.attention_exact(case)
    G = case.n_q_heads // case.n_kv_heads
    for h in range(case.n_q_heads):
        np.testing.assert_allclose(out[0, h], v[h // G, 0], rtol=1e-13)
    case.q_f32[:] = 0
    out = oracle.attention_exact(case)
    for t in (1, 17, 40, 49):
        keys = brute_force_set(t, 2, 1)
        for h in range(case.n_q_heads):
            np.testing.assert_allclose(out[t, h], v[h // G, keys].mean(axis=0), rtol=1e-12)


def expand_to_mha(case):
    """Same problem with one KV head per query head (KV head copied G times)."""
    G = case.n_q_heads // case.n_kv_heads
    mha = small_case(n=case.n_tokens, hq=case.n_q_heads, hkv=case.n_q_heads,
                     W=case.window_blocks, S=case.sink_blocks)
    for name in ("k_pool", "v_pool", "k_scale", "v_scale"):
        setattr(mha, name, np.repeat(getattr(case, name), G, axis=2))
    mha.page_table = case.page_table.copy()
    mha.q_f32, mha.q_bf16 = case.q_f32.copy(), case.q_bf16.copy()
    return mha


def test_gqa_equals_mha_with_repeated_kv():
    case = small_case(n=60, hq=8, hkv=2, W=2, S=1)
    mha = expand_to_mha(case)
    np.testing.assert_array_equal(oracle.attention_exact(case), oracle.attention_exact(mha))
    np.testing.assert_array_equal(oracle.attention_int8_mirror(case),
                                  oracle.attention_int8_mirror(mha))
    # a different head->KV-head mapping must change the result
    swapped = expand_to_mha(case)
    swapped.k_pool = case.k_pool[:, :, np.tile(np.arange(2), 4)]
    assert not np.allclose(oracle.attention_exact(swapped), oracle.attention_exact(case))


def test_page_table_permutation_invariance():
    case = small_case(n=90, W=3, S=1, extra_pool_frac=0.5)
    ident = small_case(n=90, W=3, S=1)
    nb = case.n_blocks
    for name in ("k_pool", "v_pool", "k_scale", "v_scale"):
        setattr(ident, name, getattr(case, name)[case.page_table].copy())
    ident.page_table = np.arange(nb, dtype=np.int32)
    ident.q_f32, ident.q_bf16 = case.q_f32, case.q_bf16
    np.testing.assert_array_equal(oracle.attention_exact(case), oracle.attention_exact(ident))
    np.testing.assert_array_equal(oracle.attention_int8_mirror(case),
                                  oracle.attention_int8_mirror(ident))


def test_scale_trade_between_k_scale_and_softmax_scale():
    case = small_case(n=40, W=1, S=1)
    ref = oracle.attention_exact(case)
    case.k_scale = case.k_scale * 4
    case.softmax_scale /= 4
    np.testing.assert_allclose(oracle.attention_exact(case), ref, rtol=1e-12)


# ---------------------------------------------------------------- mode (b)

def put_q_on_grid(case, seed=0):
    """Q rows whose per-row int8 codes reproduce them exactly (step 1/64)."""
    rng = np.random.default_rng(seed)
    c = rng.integers(-127, 128, size=case.q_f32.shape).astype(np.int8)
    c[..., 3] = 127
    case.q_f32 = c.astype(np.float32) / np.float32(64)
    return case


@pytest.mark.parametrize("W,S", [(0, 0), (2, 1), (1, 3)])
def test_mirror_without_p_quant_equals_exact_on_grid(W, S):
    case = put_q_on_grid(small_case(n=70, W=W, S=S))
    np.testing.assert_allclose(oracle.attention_int8_mirror(case, quantize_p=False),
                               oracle.attention_exact(case), rtol=1e-10, atol=1e-13)


def test_mirror_row0_is_v0():
    case = small_case(n=20, W=0)
    k, v = contiguous_kv(case)
    out = oracle.attention_int8_mirror(case)
    for h in range(case.n_q_heads):
        np.testing.assert_allclose(out[0, h], v[h // 2, 0], rtol=1e-13)


def test_mirror_uniform_blocks_are_exact():
    """Within each 16-key block all keys share K codes and scales, so every
    P' of a block is equal, every code is 127, and P quantization is exact;
    a per-row (rather than per-block) code would not be."""
    case = put_q_on_grid(small_case(n=64, hq=2, hkv=1, W=0, seed=9))
    for p in range(case.n_pool_pages):
        case.k_pool[p, :] = case.k_pool[p, 0]
        case.k_scale[p, :] = case.k_scale[p, 0]
        case.v_scale[p, :] = case.v_scale[p, 0] * (1 + 3 * p)
    case.k_pool[case.page_table[1]] = -case.k_pool[case.page_table[0]]  # blocks far apart
    b = oracle.attention_int8_mirror(case)
    a = oracle.attention_exact(case)
    last = [15, 31, 47, 63]
    # the only difference left is the float32 rounding of each block max
    np.testing.assert_allclose(b[last], a[last], rtol=0, atol=2e-7 * np.abs(a[last]).max())
    # a single code per row (max over all blocks) would be off by far more
    assert np.abs(b[last] - a[last]).max() < 1e-5 * np.abs(a[last]).max()


def test_mirror_hand_worked_two_keys():
    g = json.load(open(os.path.join(GOLDEN, "two_key_block.json")))
    case = workloads.make_case(n_tokens=2, n_q_heads=1, n_kv_heads=1, window_blocks=0,
                               sink_blocks=0, seed=1, poison_unused=False)
    case.q_f32[:] = 0
    case.q_f32[1, 0, 0] = np.float32(127 / 64)
    case.q_f32[0, 0, 0] = np.float32(1.0)
    case.k_pool[:] = 0
    p0 = case.page_table[0]
    case.k_pool[p0, 0, 0, 0] = -127
    case.k_pool[p0, 1, 0, 0] = 0
    case.k_scale[:] = 2.0 ** -7
    case.softmax_scale = 2.0 ** -4
    case.v_pool[p0, 0, 0, :] = g["v_codes"][0]
    case.v_pool[p0, 1, 0, :] = g["v_codes"][1]
    case.v_scale[p0, 0, 0] = g["v_scales"][0]
    case.v_scale[p0, 1, 0] = g["v_scales"][1]
    out = oracle.attention_int8_mirror(case)
    P0 = math.exp(g["s0_numerator"] / g["s0_denominator"])
    l = 1.0 + P0
    ps = P0 * g["v_scales"][0] / 127
    c0, c1 = g["codes_row1"]
    expect = ps * (c0 * g["v_codes"][0] + c1 * g["v_codes"][1]) / l
    # ps comes from the float32 block max, hence rtol 1e-7
    np.testing.assert_allclose(out[1, 0], expect, rtol=1e-7)
    np.testing.assert_allclose(out[0, 0], g["row0_output"], rtol=1e-14)
    # the unquantized value differs from the quantized one (code 72 vs 71.815)
    exact = (P0 * g["v_scales"][0] * g["v_codes"][0] + g["v_scales"][1] * g["v_codes"][1]) / l
    assert abs(exact - expect) > 1e-4


def test_mirror_p_quant_error_bound():
    """|O_b - O_noquant| <= sum_j (ps_j/2)|v_j| / l  with ps_j <= max v_scale/127
    in j's block and l >= 1: a loose but oracle-independent bound."""
    case = small_case(n=100, hq=2, hkv=1, W=2, S=1, seed=21)
    b = oracle.attention_int8_mirror(case)
    nq = oracle.attention_int8_mirror(case, quantize_p=False)
    tok = np.arange(100)
    phys, slot = case.page_table[tok // 16], tok % 16
    vabs = np.abs(case.v_pool[phys, slot, 0].astype(np.float64))
    vs = case.v_scale[phys, slot, 0].astype(np.float64)
    for t in range(100):
        keys = brute_force_set(t, 2, 1)
        bound = np.zeros(256)
        for j in keys:
            blk = [k for k in keys if k // 16 == j // 16]
            bound += vs[blk].max() / 254 * vabs[j]
        for h in range(2):
            assert np.all(np.abs(b[t, h] - nq[t, h]) <= bound * (1 + 1e-9))


def test_p_block_codes():
    from oracle.reference import _quantize_p_block
    pv = np.array([[0.5, 0.25, 0.125, 0.0], [0.0, 0.0, 0.0, 0.0], [4.0, 1.0, 0.0, 4.0]])
    codes, ps = _quantize_p_block(pv)
    # multiplier 254: 0.25 -> 63.5 -> 64 (half-even), 0.125 -> 31.75 -> 32
    assert codes[0].tolist() == [127, 64, 32, 0]
    assert codes[1].tolist() == [0, 0, 0, 0] and ps[1] == 0
    # multiplier 31.75: 1.0 -> 31.75 -> 32
    assert codes[2].tolist() == [127, 32, 0, 127]
    np.testing.assert_allclose(ps[[0, 2]], [0.5 / 127, 4.0 / 127])


def test_mirror_tie_slack_covers_an_exact_tie():
    """Equal scores and v_scale(key0) = 2 v_scale(key1) put key 1's code
    argument at exactly 63.5: rint gives 64 (half-even), 63 is equally
    faithful, and the reported slack is exactly the effect of that choice."""
    case = workloads.make_case(n_tokens=2, n_q_heads=1, n_kv_heads=1, window_blocks=0,
                               sink_blocks=0, seed=1, poison_unused=False)
    case.q_f32[:] = 0
    case.k_pool[:] = 0
    p0 = case.page_table[0]
    case.v_scale[p0, 0, 0] = 2.0 ** -6
    case.v_scale[p0, 1, 0] = 2.0 ** -7
    out, slack = oracle.attention_int8_mirror(case, tie_slack=True)
    v1 = np.abs(case.v_pool[p0, 1, 0].astype(np.float64))
    ps = 2.0 ** -6 / 127
    np.testing.assert_allclose(slack[1, 0], ps * v1 / 2.0, rtol=1e-12)
    assert np.all(slack[0, 0] == 0)
    v0 = case.v_pool[p0, 0, 0].astype(np.float64)
    vv1 = case.v_pool[p0, 1, 0].astype(np.float64)
    np.testing.assert_allclose(out[1, 0], ps * (127 * v0 + 64 * vv1) / 2.0, rtol=1e-12)
    # output without the slack request is the same array
    np.testing.assert_array_equal(oracle.attention_int8_mirror(case), out)


def test_mirror_tie_slack_is_small_on_random_inputs():
    """Near-tie codes are a small share, so the slack stays far below the
    2e-3 * max|O| bar except in short rows where one code weighs a lot."""
    case = small_case(n=300, hq=4, hkv=2, W=4, S=1, seed=33)
    out, slack = oracle.attention_int8_mirror(case, tie_slack=True)
    mo = np.abs(out).max()
    assert np.mean(slack) < 1e-4 * mo
    assert np.median(slack) == 0.0
    assert np.mean(slack[200:] > 0) < 0.4


def test_p_block_codes_for_tiny_block_max():
    """Codes depend only on P'/max: a block scaled by 2^-124 (still a normal
    float32, but 127/max overflows) keeps the codes of the unscaled block."""
    from oracle.reference import _quantize_p_block
    pv = np.array([[0.5, 0.25, 0.125, 0.0]])
    c1, ps1 = _quantize_p_block(pv)
    c2, ps2 = _quantize_p_block(pv * 2.0 ** -124)
    assert np.array_equal(c1, c2)
    assert np.all(np.isfinite(c2)) and ps2[0] > 0
