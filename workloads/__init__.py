"""Seeded synthetic inputs for windowed int8 paged prefill attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the CPU oracle and the HIP path can take their
inputs from it without sharing any of the method.

The pages ("perf(qwen35): int8 tensor-core prefill attention for Qwythos",
sections "Summary" and "Why the attention, and why tensor cores") measure
whole-model prefill of a 9B model on held-out prompts.  Neither the weights nor
the prompts exist here, so seeded tensors with the pages' shapes stand in for
them: head_dim 256, GQA-4, 16-token int8 KV pages with per-token scales, a
default window of 256 blocks plus one sink block, contexts 4k / 32k / 64k.

Layouts (all host numpy arrays, C-contiguous):
  q_bf16      uint16 [n_tokens][n_q_heads][256]   bf16 bit patterns
  q_f32       float32 same shape, the exact widening of q_bf16
  k_pool      int8   [n_pool_pages][16][n_kv_heads][256]
  v_pool      int8   same
  k_scale     float32 [n_pool_pages][16][n_kv_heads]
  v_scale     float32 same
  page_table  int32  [ceil(n_tokens / 16)]  logical block -> physical page
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 256
PAGE = 16

__all__ = ["Case", "CONFIGS", "make_config", "make_case", "make_long_row_case", "make_kv_rows", "make_decode_batch",
           "decode_row_case", "HEAD_DIM", "PAGE"]


@dataclasses.dataclass
class Case:
    name: str
    n_tokens: int
    n_q_heads: int
    n_kv_heads: int
    window_blocks: int
    sink_blocks: int
    softmax_scale: float
    out_dtype: str            # "f32" or "bf16"
    q_bf16: np.ndarray
    q_f32: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray
    page_table: np.ndarray
    seed: int

    @property
    def n_pool_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def n_blocks(self) -> int:
        return (self.n_tokens + PAGE - 1) // PAGE


def _round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-half-to-even (input generation only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_case(
    *,
    n_tokens: int,
    n_q_heads: int,
    n_kv_heads: int,
    window_blocks: int,
    sink_blocks: int,
    seed: int,
    name: str = "custom",
    softmax_scale: float = 1.0 / 16.0,
    out_dtype: str = "bf16",
    scale_lo: float = 0.005,
    scale_hi: float = 0.02,
    log_uniform_scales: bool = False,
    extra_pool_frac: float = 0.0,
    q_outlier_frac: float = 0.0,
    k_saturated_frac: float = 0.0,
    poison_unused: bool = True,
) -> Case:
    """Draw one seeded case.

    Draw order is fixed: Q, K, V, k_scale, v_scale, page permutation, then the
    outlier selections (Q outlier rows/channels, saturated K tokens, signs).
    Unused pool slots (pages not in the table, and the tail slots of a partial
    last page) get NaN scales, so any stray read of them poisons the output.
    """
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    rng = np.random.default_rng(seed)
    n_blocks = (n_tokens + PAGE - 1) // PAGE
    n_pool = n_blocks + int(round(extra_pool_frac * n_blocks))

    q = rng.standard_normal((n_tokens, n_q_heads, HEAD_DIM), dtype=np.float32)
    k_pool = rng.integers(-127, 128, size=(n_pool, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    v_pool = rng.integers(-127, 128, size=(n_pool, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    if log_uniform_scales:
        lo, hi = math.log(scale_lo), math.log(scale_hi)
        k_scale = np.exp(rng.uniform(lo, hi, size=(n_pool, PAGE, n_kv_heads))).astype(np.float32)
        v_scale = np.exp(rng.uniform(lo, hi, size=(n_pool, PAGE, n_kv_heads))).astype(np.float32)
    else:
        k_scale = rng.uniform(scale_lo, scale_hi, size=(n_pool, PAGE, n_kv_heads)).astype(np.float32)
        v_scale = rng.uniform(scale_lo, scale_hi, size=(n_pool, PAGE, n_kv_heads)).astype(np.float32)
    perm = rng.permutation(n_pool).astype(np.int32)
    page_table = np.ascontiguousarray(perm[:n_blocks])

    if q_outlier_frac > 0.0:
        n_rows = n_tokens * n_q_heads
        n_out = int(math.ceil(q_outlier_frac * n_rows))
        rows = rng.choice(n_rows, size=n_out, replace=False)
        qf = q.reshape(n_rows, HEAD_DIM)
        for r in rows:
            ch = rng.choice(HEAD_DIM, size=4, replace=False)
            qf[r, ch] *= 30.0
    if k_saturated_frac > 0.0:
        n_sat = int(math.ceil(k_saturated_frac * n_tokens))
        toks = rng.choice(n_tokens, size=n_sat, replace=False)
        signs = rng.integers(0, 2, size=(n_sat, n_kv_heads, HEAD_DIM), dtype=np.int8)
        vals = np.where(signs == 1, np.int8(127), np.int8(-127)).astype(np.int8)
        for i, t in enumerate(toks):
            k_pool[page_table[t // PAGE], t % PAGE] = vals[i]

    if poison_unused:
        used = np.zeros(n_pool, dtype=bool)
        used[page_table] = True
        k_scale[~used] = np.nan
        v_scale[~used] = np.nan
        tail = n_blocks * PAGE - n_tokens
        if tail:
            last = page_table[n_blocks - 1]
            k_scale[last, PAGE - tail:] = np.nan
            v_scale[last, PAGE - tail:] = np.nan

    q_bits = _round_to_bf16_bits(q)
    return Case(
        name=name, n_tokens=n_tokens, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
        window_blocks=window_blocks, sink_blocks=sink_blocks,
        softmax_scale=float(softmax_scale), out_dtype=out_dtype,
        q_bf16=q_bits, q_f32=_bf16_bits_to_f32(q_bits),
        k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
        page_table=page_table, seed=seed,
    )


# The five seeded workloads.  Sizes, heads, window, distributions and pool
# shapes follow the pages' shapes (hd256, GQA-4, 16-token pages, window 256
# blocks, contexts 4k/32k/64k) plus a full-causal outlier stress case.  Two
# more take the 32k workload's 16 query heads over 8 and 16 KV heads (two and
# one query heads per KV head): the same int8 work at other GQA ratios.
CONFIGS = {
    "tiny": dict(n_tokens=64, n_q_heads=2, n_kv_heads=1, window_blocks=0, sink_blocks=0,
                 seed=1001, out_dtype="f32"),
    "4k": dict(n_tokens=4096, n_q_heads=16, n_kv_heads=4, window_blocks=256, sink_blocks=1,
               seed=1002),
    "32k": dict(n_tokens=32768, n_q_heads=16, n_kv_heads=4, window_blocks=256, sink_blocks=1,
                seed=1003),
    "64k": dict(n_tokens=65536, n_q_heads=16, n_kv_heads=4, window_blocks=256, sink_blocks=1,
                seed=1004, extra_pool_frac=0.25),
    "16k_full": dict(n_tokens=16384, n_q_heads=32, n_kv_heads=8, window_blocks=0, sink_blocks=0,
                     seed=1005, scale_lo=1e-3, scale_hi=5e-2, log_uniform_scales=True,
                     q_outlier_frac=0.01, k_saturated_frac=0.02),
    "32k_gqa2": dict(n_tokens=32768, n_q_heads=16, n_kv_heads=8, window_blocks=256, sink_blocks=1,
                     seed=1006),
    "32k_mha": dict(n_tokens=32768, n_q_heads=16, n_kv_heads=16, window_blocks=256, sink_blocks=1,
                    seed=1007),
}


def make_config(name: str, seed: int | None = None) -> Case:
    kw = dict(CONFIGS[name])
    if seed is not None:
        kw["seed"] = seed
    return make_case(name=name, **kw)


def make_long_row_case(n_tokens: int, q_rows: int, n_q_heads: int, n_kv_heads: int, seed: int) -> Case:
    """A full-causal sequence whose last q_rows rows attend n_tokens keys each,
    with every V code at +127, v_scale 2^-7 on the first 64 tokens and 2^-6
    on the rest: query head 0 of those rows is all zero, so its scores are all
    equal and every P * v_scale past the first 64 keys is twice the first
    ones', which puts the int8 weights at their largest and makes the PV sums
    grow as fast as they can; the other heads are N(0,1) rounded to bf16.
    Only the last q_rows rows of Q are drawn; the rest stay zero, and the Q
    arrays are allocated lazily (np.zeros), so a long sequence costs little
    memory.  Draw order: Q rows, K codes, k_scale, page permutation."""
    rng = np.random.default_rng(seed)
    n_blocks = (n_tokens + PAGE - 1) // PAGE
    q = rng.standard_normal((q_rows, n_q_heads, HEAD_DIM), dtype=np.float32)
    q[:, 0] = 0.0
    k_pool = rng.integers(-127, 128, size=(n_blocks, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    k_scale = rng.uniform(0.005, 0.02, size=(n_blocks, PAGE, n_kv_heads)).astype(np.float32)
    page_table = rng.permutation(n_blocks).astype(np.int32)
    v_pool = np.full((n_blocks, PAGE, n_kv_heads, HEAD_DIM), 127, dtype=np.int8)
    v_scale = np.full((n_blocks, PAGE, n_kv_heads), 2.0 ** -6, dtype=np.float32)
    v_scale[page_table[:4]] = 2.0 ** -7
    q_bits = np.zeros((n_tokens, n_q_heads, HEAD_DIM), dtype=np.uint16)
    q_f32 = np.zeros((n_tokens, n_q_heads, HEAD_DIM), dtype=np.float32)
    q_bits[n_tokens - q_rows:] = _round_to_bf16_bits(q)
    q_f32[n_tokens - q_rows:] = _bf16_bits_to_f32(q_bits[n_tokens - q_rows:])
    return Case(name="long_row", n_tokens=n_tokens, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, window_blocks=0,
                sink_blocks=0, softmax_scale=1.0 / 16.0, out_dtype="f32", q_bf16=q_bits, q_f32=q_f32,
                k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale, page_table=page_table, seed=seed)


def make_kv_rows(n_tokens: int, n_kv_heads: int, n_pool_pages: int, seed: int):
    """Seeded inputs of the KV-pool writer.

    Returns (k_bf16, v_bf16, k_f32, v_f32, slots, k_pool, v_pool, k_scale, v_scale):
    K and V rows drawn N(0, 1) and rounded to bf16 (bit patterns uint16, and
    their exact float32 widening), [n_tokens][n_kv_heads][256]; slots, int32
    [n_tokens], distinct pool slots in seeded random order; and a pool to write
    into whose contents are random codes and scales, so untouched rows show.
    Draw order: K, V, slots, pool codes, pool scales.
    """
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_tokens, n_kv_heads, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((n_tokens, n_kv_heads, HEAD_DIM), dtype=np.float32)
    n_slots = n_pool_pages * PAGE
    if n_tokens > n_slots:
        raise ValueError("more tokens than pool slots")
    slots = rng.permutation(n_slots)[:n_tokens].astype(np.int32)
    k_pool = rng.integers(-127, 128, size=(n_pool_pages, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    v_pool = rng.integers(-127, 128, size=(n_pool_pages, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    k_scale = rng.uniform(0.005, 0.02, size=(n_pool_pages, PAGE, n_kv_heads)).astype(np.float32)
    v_scale = rng.uniform(0.005, 0.02, size=(n_pool_pages, PAGE, n_kv_heads)).astype(np.float32)
    kb, vb = _round_to_bf16_bits(k), _round_to_bf16_bits(v)
    return (kb, vb, _bf16_bits_to_f32(kb), _bf16_bits_to_f32(vb), slots, k_pool, v_pool, k_scale, v_scale)


@dataclasses.dataclass
class DecodeBatch:
    """Inputs of one decode step: sequence b has seq_lens[b] tokens in the pool and
    its last position is the query q[b]."""
    n_q_heads: int
    n_kv_heads: int
    window_blocks: int
    sink_blocks: int
    softmax_scale: float
    q_bf16: np.ndarray        # uint16 [batch][n_q_heads][256]
    q_f32: np.ndarray         # float32, the exact widening
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray
    page_tables: np.ndarray   # int32 [batch][max_blocks]; -1 past each sequence's last block
    seq_lens: np.ndarray      # int32 [batch]


def make_decode_batch(seq_lens, n_q_heads: int, n_kv_heads: int, window_blocks: int, sink_blocks: int,
                      seed: int, max_blocks: int | None = None, owned_pages: bool = False,
                      softmax_scale: float = 1.0 / 16.0) -> DecodeBatch:
    """Seeded decode inputs.  Draw order: Q, pool codes (K, V), scales (K, V), page maps.

    Page 0 of the pool is never mapped and has NaN scales, so that a page
    table entry pointed at it (as the tests do for blocks a query must not
    read) poisons any read of it.  By default every sequence maps its blocks
    to a seeded random choice of distinct pages out of pages 1 .. max_blocks
    (sequences may share pages).  With owned_pages, every block of every
    sequence gets a page of its own, sequence b's pages a contiguous range of
    the pool in seeded random order (a per-sequence allocator), so a decode
    step streams exactly the pages it reads and no two sequences share one."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    batch = len(seq_lens)
    rng = np.random.default_rng(seed)
    need = [(int(L) + PAGE - 1) // PAGE for L in seq_lens]
    max_blocks = max_blocks or max(max(need), 1)
    q = rng.standard_normal((batch, n_q_heads, HEAD_DIM), dtype=np.float32)
    n_pool = 1 + (sum(need) if owned_pages else max_blocks)
    k_pool = rng.integers(-127, 128, size=(n_pool, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    v_pool = rng.integers(-127, 128, size=(n_pool, PAGE, n_kv_heads, HEAD_DIM), dtype=np.int8)
    k_scale = rng.uniform(0.005, 0.02, size=(n_pool, PAGE, n_kv_heads)).astype(np.float32)
    v_scale = rng.uniform(0.005, 0.02, size=(n_pool, PAGE, n_kv_heads)).astype(np.float32)
    k_scale[0] = np.nan
    v_scale[0] = np.nan
    tables = np.full((batch, max_blocks), -1, dtype=np.int32)
    if owned_pages:
        nxt = 1
        for b in range(batch):
            tables[b, :need[b]] = rng.permutation(need[b]).astype(np.int32) + nxt
            nxt += need[b]
    else:
        for b in range(batch):
            tables[b, :need[b]] = rng.permutation(n_pool - 1)[:need[b]] + 1
    qb = _round_to_bf16_bits(q)
    return DecodeBatch(n_q_heads, n_kv_heads, window_blocks, sink_blocks, softmax_scale, qb,
                       _bf16_bits_to_f32(qb), k_pool, v_pool, k_scale, v_scale, tables, seq_lens)


def decode_row_case(batch: DecodeBatch, b: int) -> Case:
    """Sequence b of a decode batch as a prefill case whose row seq_lens[b]-1 is
    the decode query (all other rows zero), for evaluating the oracle there."""
    L = int(batch.seq_lens[b])
    qf = np.zeros((L, batch.n_q_heads, HEAD_DIM), dtype=np.float32)
    qb = np.zeros((L, batch.n_q_heads, HEAD_DIM), dtype=np.uint16)
    qf[L - 1], qb[L - 1] = batch.q_f32[b], batch.q_bf16[b]
    table = batch.page_tables[b, :(L + PAGE - 1) // PAGE].copy()
    return Case(name=f"decode{b}", n_tokens=L, n_q_heads=batch.n_q_heads, n_kv_heads=batch.n_kv_heads,
                window_blocks=batch.window_blocks, sink_blocks=batch.sink_blocks,
                softmax_scale=batch.softmax_scale, out_dtype="f32", q_bf16=qb, q_f32=qf, k_pool=batch.k_pool,
                v_pool=batch.v_pool, k_scale=batch.k_scale, v_scale=batch.v_scale, page_table=table, seed=0)
