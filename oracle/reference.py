"""CPU oracle for windowed int8 paged prefill attention (head_dim 256).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module; the product path never does.  It
shares no code, table or helper with the HIP library.

Plain, slow, obviously-correct numpy.  Floating point is fp64 except where the
method turns a float into an integer code (Q and P quantization): there the
decision is taken in float32, the precision the kernel takes it in.

Sources (the pages):
  [465/Why]  "perf(qwen35): int8 tensor-core prefill attention for Qwythos",
             section "Why the attention, and why tensor cores": pages are 16
             tokens, rows token-major with stride n_kv_heads*head_dim; Q is
             quantized with one scale per query row, QK^T runs int8 x int8 ->
             int32 and the row Q scale, the per-token K scale and the softmax
             scale are applied to the int32; the per-token V scale is folded
             into P, P is quantized and PV runs int8; the mask is causal plus
             sink/window, block-granular, with n_blk_q = (t+16)/16 constant
             over a 16-row query tile; the online softmax is the usual one.
  [465/Rel]  same page, section "Relation to open PRs": a window of
             win_blocks <= 0 means full causal attention; GQA-4 at hd256.
  [463/Sum]  "perf(qwen35): fp16 shared-memory tiles for windowed prefill
             attention", sections "Summary"/"Proof of speedup": the window is
             the StreamingLLM one; setting the window to 0 disables it.

Readings taken where the pages are silent (each listed in the design notes):
  * window start rsb(t) = max(0, n_blk_q(t) - W), n_blk_q(t) = t//16 + 1:
    the window is the last W key blocks including the current partial one;
  * sink = the first S key blocks, joined with the window as a set;
  * W <= 0: full causal, S ignored;  the causal bound is inclusive (j <= t)
    and prefill starts at position 0;
  * Q row = one (token, head) pair over the 256 channels; scale = amax/127,
    codes = round-half-even(q * (127/amax)) clamped to +-127; amax = 0 gives
    scale 0 and all-zero codes;
  * P is quantized per (row, 16-key block): the block max of P*v_scale maps
    to 127; masked keys are excluded and contribute nothing;
  * the softmax denominator is the sum of the unquantized P;
  * the KV head of query head h is h // (n_q_heads // n_kv_heads).

Parity status: every function here is pinned by tests (closed forms, library
special cases, brute force, hand-worked values); see tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 256
PAGE = 16

__all__ = [
    "window_start_block", "attended_mask", "mask_counts", "quantize_q_rows", "kv_write_i8",
    "dequant_keys_values", "attention_exact", "attention_int8_mirror",
    "tile_rows", "HEAD_DIM", "PAGE",
]


# ----------------------------------------------------------------------------
# The attended-key set  [465/Why], [465/Rel], [463/Sum]
# ----------------------------------------------------------------------------

def window_start_block(t: np.ndarray | int, window_blocks: int):
    """rsb(t) = max(0, n_blk_q - W) with n_blk_q = (t + 16) // 16."""
    n_blk_q = (np.asarray(t) + PAGE) // PAGE
    return np.maximum(0, n_blk_q - window_blocks)


def attended_mask(t_rows: np.ndarray, keys: np.ndarray, window_blocks: int,
                  sink_blocks: int) -> np.ndarray:
    """Boolean [len(t_rows)][len(keys)]: is key j in A(t)?

    A(t) = { j <= t : W <= 0  or  j//16 < S  or  j//16 >= rsb(t) }.
    """
    t = np.asarray(t_rows, dtype=np.int64)[:, None]
    j = np.asarray(keys, dtype=np.int64)[None, :]
    causal = j <= t
    if window_blocks <= 0:
        return causal
    blk = j // PAGE
    rsb = window_start_block(t, window_blocks)
    return causal & ((blk < sink_blocks) | (blk >= rsb))


def mask_counts(n_tokens: int, window_blocks: int, sink_blocks: int) -> np.ndarray:
    """|A(t)| for every query row t, by enumerating the set definition."""
    out = np.zeros(n_tokens, dtype=np.int64)
    for t0 in range(0, n_tokens, PAGE):
        rows = np.arange(t0, min(t0 + PAGE, n_tokens))
        keys = np.arange(0, rows[-1] + 1)
        out[rows] = attended_mask(rows, keys, window_blocks, sink_blocks).sum(axis=1)
    return out


# ----------------------------------------------------------------------------
# Q row quantization  [465/Why]: one scale per query row
# ----------------------------------------------------------------------------

def quantize_q_rows(q: np.ndarray):
    """q [..., 256] (values exactly representable in float32) ->
    (codes int8 [..., 256], scale float32 [...]).

    Taken in float32, as the kernel takes it:
      amax = max |q|;  inv = 127 / amax;  code = clip(rint(q * inv), -127, 127);
      scale = amax / 127;  amax == 0  ->  scale 0, codes 0.
    np.rint rounds half to even.
    """
    q32 = np.asarray(q, dtype=np.float32)
    amax = np.max(np.abs(q32), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(127.0) / safe).astype(np.float32)
    prod = (q32 * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    codes[~nz] = 0
    scale = np.where(nz, (amax / np.float32(127.0)).astype(np.float32), np.float32(0.0))
    return codes, scale.astype(np.float32)


# ----------------------------------------------------------------------------
# KV-pool writer: the pool the pages read, filled row by row  [465/Why]
# ----------------------------------------------------------------------------

def kv_write_i8(k: np.ndarray, v: np.ndarray, slots: np.ndarray, k_pool: np.ndarray,
                v_pool: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray):
    """Quantize K and V rows into copies of the int8 pool.

    k, v: [n_tokens][n_kv_heads][256] (float32-representable values);
    slots: [n_tokens] ints, slot = physical page * 16 + position in the page;
    pools [P][16][Hkv][256] int8, scales [P][16][Hkv] float32.

    The page gives the pool's layout (16-token pages, one scale per token and
    KV head) but not how it is filled; each (token, head) row is quantized
    with the per-row formula the page gives for Q (quantize_q_rows), and a
    slot outside [0, 16 * P) is skipped.  Returns the four updated arrays.
    """
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    k_scale, v_scale = k_scale.copy(), v_scale.copy()
    n_pages = k_pool.shape[0]
    kc, ks = quantize_q_rows(k)
    vc, vs = quantize_q_rows(v)
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if not 0 <= slot < n_pages * PAGE:
            continue
        page, pos = divmod(slot, PAGE)
        k_pool[page, pos] = kc[t]
        v_pool[page, pos] = vc[t]
        k_scale[page, pos] = ks[t]
        v_scale[page, pos] = vs[t]
    return k_pool, v_pool, k_scale, v_scale


# ----------------------------------------------------------------------------
# Paged pool access  [465/Why]: 16-token pages, rows token-major
# ----------------------------------------------------------------------------

def _gather(pool: np.ndarray, page_table: np.ndarray, keys: np.ndarray, kvh: int):
    """Rows of a [P][16][Hkv][...] pool for logical key indices `keys`."""
    phys = page_table[keys // PAGE]
    return pool[phys, keys % PAGE, kvh]


def dequant_keys_values(case_arrays, keys: np.ndarray, kvh: int):
    """Kd[j] = k_i8[j] * k_scale[j], Vd[j] = v_i8[j] * v_scale[j] in fp64."""
    k_pool, v_pool, k_scale, v_scale, page_table = case_arrays
    ki = _gather(k_pool, page_table, keys, kvh).astype(np.float64)
    vi = _gather(v_pool, page_table, keys, kvh).astype(np.float64)
    ks = _gather(k_scale, page_table, keys, kvh).astype(np.float64)
    vs = _gather(v_scale, page_table, keys, kvh).astype(np.float64)
    return ki * ks[:, None], vi * vs[:, None]


def tile_rows(n_tokens: int, tile: int) -> np.ndarray:
    return np.arange(tile * PAGE, min((tile + 1) * PAGE, n_tokens))


def _tile_keys(rows: np.ndarray, window_blocks: int, sink_blocks: int):
    """All keys any row of the tile attends, and the [rows][keys] mask."""
    cand = np.arange(0, rows[-1] + 1)
    m = attended_mask(rows, cand, window_blocks, sink_blocks)
    keep = m.any(axis=0)
    return cand[keep], m[:, keep]


def _arrays(case):
    return (case.k_pool, case.v_pool, case.k_scale, case.v_scale, case.page_table)


# ----------------------------------------------------------------------------
# Mode (a): exact masked softmax attention over dequantized K/V, fp64
# ----------------------------------------------------------------------------

def attention_exact(case, tiles=None) -> np.ndarray:
    """O[t,h] = sum_{j in A(t)} softmax_j(alpha * q[t,h] . Kd[j]) Vd[j].

    q is the bf16 input widened to fp64 (unquantized); two-pass softmax with
    the true row max.  Returns fp64 [n_tokens][n_q_heads][256]; rows of tiles
    not listed in `tiles` are left as NaN.
    """
    N, Hq, Hkv = case.n_tokens, case.n_q_heads, case.n_kv_heads
    G = Hq // Hkv
    alpha = float(case.softmax_scale)
    out = np.full((N, Hq, HEAD_DIM), np.nan)
    arrays = _arrays(case)
    n_tiles = (N + PAGE - 1) // PAGE
    for tile in (range(n_tiles) if tiles is None else tiles):
        rows = tile_rows(N, tile)
        keys, mask = _tile_keys(rows, case.window_blocks, case.sink_blocks)
        for kvh in range(Hkv):
            Kd, Vd = dequant_keys_values(arrays, keys, kvh)
            for h in range(kvh * G, (kvh + 1) * G):
                q = case.q_f32[rows, h].astype(np.float64)
                s = alpha * (q @ Kd.T)
                s = np.where(mask, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.where(mask, np.exp(s - m), 0.0)
                out[rows, h] = (p @ Vd) / p.sum(axis=1, keepdims=True)
    return out


# ----------------------------------------------------------------------------
# Mode (b): mirror of the int8 scheme
# ----------------------------------------------------------------------------

# A code is "near a tie" when its float32 argument x = P' * 127/mx lies within
# TIE_WINDOW * x of k + 1/2.  At float32 precision either rounding of such a
# code is a faithful result of the method: the arguments of an independent
# float32 computation differ from these by at most about 2e-6 * x, and
# 7.3e-6 * x with scores near 50 (outlier rows), so the window is about twice
# the largest of those.  The slack is a diagnostic; the acceptance bar does
# not use it.
TIE_WINDOW = 2.0 ** -16


def _quantize_p_block(pv: np.ndarray, with_ties: bool = False):
    """Per-row int8 code of one 16-key block of P' = P * v_scale (>= 0).

    Decision in float32: mx = max P'; code = clip(rint(P' * (127/mx)), +-127);
    step ps = mx / 127.  Rows with no attended key (mx == 0) get code 0.
    With with_ties, also returns the boolean mask of near-tie codes.
    """
    p32 = pv.astype(np.float32)
    mx = p32.max(axis=1)
    nz = mx > 0
    # The code depends only on P'/max.  Blocks whose max is so small that
    # 127/max would overflow float32 are first scaled by 2^64 (exact).
    tiny = nz & (mx < np.float32(2.0 ** -60))
    up = np.where(tiny, np.float32(2.0 ** 64), np.float32(1.0)).astype(np.float32)
    p32s = (p32 * up[:, None]).astype(np.float32)
    mxs = (mx * up).astype(np.float32)
    inv = (np.float32(127.0) / np.where(nz, mxs, np.float32(1.0))).astype(np.float32)
    x = (p32s * inv[:, None]).astype(np.float32)
    codes = np.clip(np.rint(x), -127, 127)
    codes[~nz] = 0.0
    ps = np.where(nz, mx.astype(np.float64) / 127.0, 0.0)
    if not with_ties:
        return codes.astype(np.float64), ps
    xd = x.astype(np.float64)
    ties = (np.abs(xd - (np.floor(xd) + 0.5)) <= TIE_WINDOW * xd) & nz[:, None]
    return codes.astype(np.float64), ps, ties


def attention_int8_mirror(case, tiles=None, quantize_p: bool = True,
                          q_codes=None, q_scale=None, tie_slack: bool = False):
    """Mirror of the int8 path, fp64 except the quantization decisions.

      1. Q rows quantized (quantize_q_rows).
      2. acc = q_i8 . k_i8, exact integers.
      3. s = acc * q_scale[row] * k_scale[key] * alpha.
      4. m = max over A(t); P = exp(s - m); l = sum over A(t) of P.
      5. P' = P * v_scale[key]; per (row, 16-key block) P' -> int8 codes with
         step ps = blockmax/127 (quantize_p=False keeps P' unquantized).
      6. O = sum over blocks of ps * (codes . v_i8), divided by l.
    Returns fp64 [n_tokens][n_q_heads][256]; unlisted tiles stay NaN.
    With tie_slack, also returns slack[t,h,d] = sum over near-tie codes j of
    ps_j * |v_i8[j,d]| / l: the most that re-rounding those codes the other
    way can move the output.
    """
    N, Hq, Hkv = case.n_tokens, case.n_q_heads, case.n_kv_heads
    G = Hq // Hkv
    alpha = float(case.softmax_scale)
    slack = np.full((N, Hq, HEAD_DIM), np.nan) if tie_slack else None
    if q_codes is None:
        q_codes, q_scale = quantize_q_rows(case.q_f32)
    out = np.full((N, Hq, HEAD_DIM), np.nan)
    n_tiles = (N + PAGE - 1) // PAGE
    for tile in (range(n_tiles) if tiles is None else tiles):
        rows = tile_rows(N, tile)
        keys, mask = _tile_keys(rows, case.window_blocks, case.sink_blocks)
        kblk = keys // PAGE
        blocks = np.unique(kblk)
        for kvh in range(Hkv):
            ki = _gather(case.k_pool, case.page_table, keys, kvh).astype(np.float64)
            vi = _gather(case.v_pool, case.page_table, keys, kvh).astype(np.float64)
            ks = _gather(case.k_scale, case.page_table, keys, kvh).astype(np.float64)
            vs = _gather(case.v_scale, case.page_table, keys, kvh).astype(np.float64)
            for h in range(kvh * G, (kvh + 1) * G):
                qi = q_codes[rows, h].astype(np.float64)
                qs = q_scale[rows, h].astype(np.float64)
                acc = qi @ ki.T
                s = acc * qs[:, None] * ks[None, :] * alpha
                s = np.where(mask, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.where(mask, np.exp(s - m), 0.0)
                l = p.sum(axis=1)
                pv = np.where(mask, p * vs[None, :], 0.0)
                o = np.zeros((len(rows), HEAD_DIM))
                sl = np.zeros((len(rows), HEAD_DIM))
                for b in blocks:
                    cols = kblk == b
                    if quantize_p and tie_slack:
                        codes, ps, ties = _quantize_p_block(pv[:, cols], with_ties=True)
                        o += ps[:, None] * (codes @ vi[cols])
                        sl += ps[:, None] * (ties.astype(np.float64) @ np.abs(vi[cols]))
                    elif quantize_p:
                        codes, ps = _quantize_p_block(pv[:, cols])
                        o += ps[:, None] * (codes @ vi[cols])
                    else:
                        o += pv[:, cols] @ vi[cols]
                out[rows, h] = o / l[:, None]
                if tie_slack:
                    slack[rows, h] = sl / l[:, None]
    return (out, slack) if tie_slack else out
