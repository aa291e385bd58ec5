"""Python binding of libwpa.so: windowed int8 paged prefill attention on MI355X.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; PyTorch provides device memory and the current stream.  There is no
CPU fallback: if the built library is missing, importing this package raises.

Entry points mirror the C ABI in include/wpa.h:
    quantize_q_rows(q, q_i8=None, q_scale=None)      -> (q_i8, q_scale)
    prefill_attn_i8(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
                    window_blocks, sink_blocks, softmax_scale, out=None,
                    out_dtype=torch.bfloat16)          -> out
    mask_counts(n_tokens, window_blocks, sink_blocks, counts=None, device=None) -> counts
    kv_write_i8(k, v, slots, k_pool, v_pool, k_scale, v_scale)  (writes the pools in place)
    prefill_attn_i8_chunk(q_start, q_i8, q_scale, ...same as prefill_attn_i8...) -> out
    mask_counts_chunk(q_start, n_tokens, window_blocks, sink_blocks, counts=None, device=None) -> counts
    prefill_attn_fused_q(q, k_pool, ...same as prefill_attn_i8..., q_start=0) -> out   (bf16 Q, quantized in-kernel)
    decode_attn_i8(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_tables, seq_lens,
                   window_blocks, sink_blocks, softmax_scale, out=None, out_dtype=torch.bfloat16,
                   workspace=None)                     -> out
    decode_attn_i8_noalloc(...same as decode_attn_i8 without workspace...) -> out
                                                       (the library's fixed scratch; nothing allocated by the call)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["quantize_q_rows", "prefill_attn_i8", "prefill_attn_i8_chunk", "prefill_attn_fused_q", "mask_counts",
           "mask_counts_chunk",
           "kv_write_i8", "decode_attn_i8", "decode_attn_i8_noalloc", "decode_workspace_bytes", "NOALLOC_SCRATCH_BYTES",
           "lib", "LIB_PATH",
           "HEAD_DIM", "PAGE_TOKENS", "WpaError"]

HEAD_DIM = 256
PAGE_TOKENS = 16
NOALLOC_SCRATCH_BYTES = 64 << 20  # WPA_NOALLOC_SCRATCH_BYTES
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwpa.so")

WPA_F32, WPA_BF16 = 0, 1


class WpaError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run windowed_int8_paged_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.wpa_quantize_q_rows.argtypes = [vp, ci, ci, ci, vp, vp, vp]
    L.wpa_quantize_q_rows.restype = ci
    L.wpa_prefill_attn_i8.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_prefill_attn_i8.restype = ci
    L.wpa_mask_counts.argtypes = [ci, ci, ci, vp, vp]
    L.wpa_mask_counts.restype = ci
    L.wpa_prefill_attn_i8_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_prefill_attn_i8_chunk.restype = ci
    L.wpa_mask_counts_chunk.argtypes = [ci, ci, ci, ci, vp, vp]
    L.wpa_mask_counts_chunk.restype = ci
    L.wpa_prefill_attn_fused_q.argtypes = [vp, ci, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_prefill_attn_fused_q.restype = ci
    L.wpa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    L.wpa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.wpa_decode_attn_i8.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, ci, vp, ci, ci, ci, ci, ci, cf, vp,
                                     ctypes.c_size_t, vp, ci, vp]
    L.wpa_decode_attn_i8.restype = ci
    L.wpa_decode_attn_i8_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, ci, vp, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_decode_attn_i8_noalloc.restype = ci
    L.wpa_kv_write_i8.argtypes = [vp, vp, ci, ci, ci, vp, ci, vp, vp, vp, vp, vp]
    L.wpa_kv_write_i8.restype = ci
    L.wpa_status_string.argtypes = [ci]
    L.wpa_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


def _check(status: int):
    if status != 0:
        raise WpaError(lib.wpa_status_string(status).decode())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def quantize_q_rows(q, q_i8=None, q_scale=None):
    """q: [n_tokens][n_q_heads][256] bf16 or f32 on the device."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    _dev(q, "q", q.dtype)
    n, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head_dim must be 256")
    if q_i8 is None:
        q_i8 = torch.empty((n, hq, d), dtype=torch.int8, device=q.device)
    if q_scale is None:
        q_scale = torch.empty((n, hq), dtype=torch.float32, device=q.device)
    _dev(q_i8, "q_i8", torch.int8, (n, hq, d))
    _dev(q_scale, "q_scale", torch.float32, (n, hq))
    _check(lib.wpa_quantize_q_rows(_ptr(q), WPA_BF16 if q.dtype == torch.bfloat16 else WPA_F32,
                                   n, hq, _ptr(q_i8), _ptr(q_scale), _stream(q.device)))
    return q_i8, q_scale


def prefill_attn_i8(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
                    window_blocks, sink_blocks, softmax_scale, out=None, out_dtype=torch.bfloat16):
    """Paged int8 prefill attention; see include/wpa.h for the definition."""
    return _prefill(None, q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
                    window_blocks, sink_blocks, softmax_scale, out, out_dtype)


def prefill_attn_i8_chunk(q_start, q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
                          window_blocks, sink_blocks, softmax_scale, out=None, out_dtype=torch.bfloat16):
    """The query rows at positions q_start .. q_start+n-1 (q_start a multiple of 16)
    over a pool holding keys 0 .. q_start+n-1; see include/wpa.h."""
    return _prefill(int(q_start), q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
                    window_blocks, sink_blocks, softmax_scale, out, out_dtype)


def prefill_attn_fused_q(q, k_pool, v_pool, k_scale, v_scale, page_table, window_blocks, sink_blocks,
                         softmax_scale, out=None, out_dtype=torch.bfloat16, q_start=0):
    """The attention of prefill_attn_i8_chunk from bf16 Q, quantized inside the attention
    kernels (bitwise the same output as quantize_q_rows + prefill_attn_i8_chunk); see include/wpa.h."""
    return _prefill(int(q_start), q, None, k_pool, v_pool, k_scale, v_scale, page_table,
                    window_blocks, sink_blocks, softmax_scale, out, out_dtype, fused=True)


def _prefill(q_start, q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
             window_blocks, sink_blocks, softmax_scale, out, out_dtype, fused=False):
    if fused:
        _dev(q_i8, "q", torch.bfloat16)
    else:
        _dev(q_i8, "q_i8", torch.int8)
    n, hq, d = q_i8.shape
    if not fused:
        _dev(q_scale, "q_scale", torch.float32, (n, hq))
    _dev(k_pool, "k_pool", torch.int8)
    n_pool, page, hkv, d2 = k_pool.shape
    if page != PAGE_TOKENS or d2 != HEAD_DIM or d != HEAD_DIM:
        raise ValueError("pool pages must be [16][n_kv_heads][256]")
    _dev(v_pool, "v_pool", torch.int8, k_pool.shape)
    _dev(k_scale, "k_scale", torch.float32, (n_pool, page, hkv))
    _dev(v_scale, "v_scale", torch.float32, (n_pool, page, hkv))
    _dev(page_table, "page_table", torch.int32)
    if page_table.numel() < ((q_start or 0) + n + PAGE_TOKENS - 1) // PAGE_TOKENS:
        raise ValueError("page_table is shorter than ceil((q_start + n_tokens)/16)")
    if out is None:
        out = torch.empty((n, hq, d), dtype=out_dtype, device=q_i8.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _dev(out, "out", out.dtype, (n, hq, d))
    common = (_ptr(q_i8), _ptr(None if fused else q_scale), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
              _ptr(page_table), n_pool)
    tail = (n, hq, hkv, int(window_blocks), int(sink_blocks), float(softmax_scale), _ptr(out),
            WPA_BF16 if out.dtype == torch.bfloat16 else WPA_F32, _stream(q_i8.device))
    if fused:
        _check(lib.wpa_prefill_attn_fused_q(_ptr(q_i8), WPA_BF16, *common[2:], q_start, *tail))
    elif q_start is None:
        _check(lib.wpa_prefill_attn_i8(*common, *tail))
    else:
        _check(lib.wpa_prefill_attn_i8_chunk(*common, q_start, *tail))
    return out


def mask_counts(n_tokens, window_blocks, sink_blocks, counts=None, device=None):
    if counts is None:
        counts = torch.empty((n_tokens,), dtype=torch.int32, device=device or "cuda")
    _dev(counts, "counts", torch.int32, (n_tokens,))
    _check(lib.wpa_mask_counts(int(n_tokens), int(window_blocks), int(sink_blocks), _ptr(counts),
                               _stream(counts.device)))
    return counts


def mask_counts_chunk(q_start, n_tokens, window_blocks, sink_blocks, counts=None, device=None):
    if counts is None:
        counts = torch.empty((n_tokens,), dtype=torch.int32, device=device or "cuda")
    _dev(counts, "counts", torch.int32, (n_tokens,))
    _check(lib.wpa_mask_counts_chunk(int(q_start), int(n_tokens), int(window_blocks), int(sink_blocks),
                                     _ptr(counts), _stream(counts.device)))
    return counts


def kv_write_i8(k, v, slots, k_pool, v_pool, k_scale, v_scale):
    """Quantize K and V rows ([n_tokens][n_kv_heads][256], bf16 or f32) into the
    int8 pools at pool slots `slots` (int32 [n_tokens], page * 16 + position);
    see include/wpa.h for the definition.  Writes the pools in place."""
    if k.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("k must be bfloat16 or float32")
    _dev(k, "k", k.dtype)
    n, hkv, d = k.shape
    if d != HEAD_DIM:
        raise ValueError("head_dim must be 256")
    _dev(v, "v", k.dtype, (n, hkv, d))
    _dev(slots, "slots", torch.int32, (n,))
    _dev(k_pool, "k_pool", torch.int8)
    n_pool = k_pool.shape[0]
    _dev(k_pool, "k_pool", torch.int8, (n_pool, PAGE_TOKENS, hkv, HEAD_DIM))
    _dev(v_pool, "v_pool", torch.int8, (n_pool, PAGE_TOKENS, hkv, HEAD_DIM))
    _dev(k_scale, "k_scale", torch.float32, (n_pool, PAGE_TOKENS, hkv))
    _dev(v_scale, "v_scale", torch.float32, (n_pool, PAGE_TOKENS, hkv))
    _check(lib.wpa_kv_write_i8(_ptr(k), _ptr(v), WPA_BF16 if k.dtype == torch.bfloat16 else WPA_F32, n, hkv,
                               _ptr(slots), n_pool, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                               _stream(k.device)))


def decode_workspace_bytes(batch, n_q_heads, max_blocks, window_blocks, sink_blocks):
    return int(lib.wpa_decode_workspace_bytes(int(batch), int(n_q_heads), int(max_blocks), int(window_blocks),
                                              int(sink_blocks)))


def decode_attn_i8(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_tables, seq_lens,
                   window_blocks, sink_blocks, softmax_scale, out=None, out_dtype=torch.bfloat16, workspace=None):
    """One query token per sequence (its last position) over the paged pool;
    see include/wpa.h.  page_tables: int32 [batch][max_blocks]; seq_lens: int32 [batch]."""
    _dev(q_i8, "q_i8", torch.int8)
    batch, hq, d = q_i8.shape
    if d != HEAD_DIM:
        raise ValueError("head_dim must be 256")
    _dev(q_scale, "q_scale", torch.float32, (batch, hq))
    _dev(k_pool, "k_pool", torch.int8)
    n_pool, page, hkv, d2 = k_pool.shape
    if page != PAGE_TOKENS or d2 != HEAD_DIM:
        raise ValueError("pool pages must be [16][n_kv_heads][256]")
    _dev(v_pool, "v_pool", torch.int8, k_pool.shape)
    _dev(k_scale, "k_scale", torch.float32, (n_pool, page, hkv))
    _dev(v_scale, "v_scale", torch.float32, (n_pool, page, hkv))
    _dev(page_tables, "page_tables", torch.int32)
    if page_tables.dim() != 2 or page_tables.shape[0] != batch:
        raise ValueError("page_tables must be [batch][max_blocks]")
    max_blocks = page_tables.shape[1]
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    need = decode_workspace_bytes(batch, hq, max_blocks, window_blocks, sink_blocks)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q_i8.device)
    _dev(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((batch, hq, d), dtype=out_dtype, device=q_i8.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _dev(out, "out", out.dtype, (batch, hq, d))
    _check(lib.wpa_decode_attn_i8(
        _ptr(q_i8), _ptr(q_scale), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), n_pool,
        _ptr(page_tables), max_blocks, _ptr(seq_lens), batch, hq, hkv, int(window_blocks), int(sink_blocks),
        float(softmax_scale), _ptr(workspace), workspace.numel(), _ptr(out),
        WPA_BF16 if out.dtype == torch.bfloat16 else WPA_F32, _stream(q_i8.device)))
    return out


def decode_attn_i8_noalloc(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_tables, seq_lens,
                           window_blocks, sink_blocks, softmax_scale, out=None, out_dtype=torch.bfloat16):
    """decode_attn_i8 with the library's fixed scratch buffer instead of a workspace
    (wpa_decode_attn_i8_noalloc; see include/wpa.h).  Calls on one GPU share that
    buffer, so calls that overlap on one GPU race."""
    _dev(q_i8, "q_i8", torch.int8)
    batch, hq, d = q_i8.shape
    if d != HEAD_DIM:
        raise ValueError("head_dim must be 256")
    _dev(q_scale, "q_scale", torch.float32, (batch, hq))
    _dev(k_pool, "k_pool", torch.int8)
    n_pool, page, hkv, d2 = k_pool.shape
    if page != PAGE_TOKENS or d2 != HEAD_DIM:
        raise ValueError("pool pages must be [16][n_kv_heads][256]")
    _dev(v_pool, "v_pool", torch.int8, k_pool.shape)
    _dev(k_scale, "k_scale", torch.float32, (n_pool, page, hkv))
    _dev(v_scale, "v_scale", torch.float32, (n_pool, page, hkv))
    _dev(page_tables, "page_tables", torch.int32)
    if page_tables.dim() != 2 or page_tables.shape[0] != batch:
        raise ValueError("page_tables must be [batch][max_blocks]")
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    if out is None:
        out = torch.empty((batch, hq, d), dtype=out_dtype, device=q_i8.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _dev(out, "out", out.dtype, (batch, hq, d))
    _check(lib.wpa_decode_attn_i8_noalloc(
        _ptr(q_i8), _ptr(q_scale), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), n_pool,
        _ptr(page_tables), page_tables.shape[1], _ptr(seq_lens), batch, hq, hkv, int(window_blocks),
        int(sink_blocks), float(softmax_scale), _ptr(out), WPA_BF16 if out.dtype == torch.bfloat16 else WPA_F32,
        _stream(q_i8.device)))
    return out

