"""C-ABI library checks that need no GPU: the built library loads, exports every
function include/wpa.h declares, and rejects invalid arguments on the host
(before any HIP call) with the documented status codes."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wpa.h")
LIB = os.path.join(ROOT, "windowed_int8_paged_amd", "libwpa.so")

OK, NULL, SHAPE, UNSUP, LAUNCH = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wpa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libwpa.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.wpa_prefill_attn_i8.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_quantize_q_rows.argtypes = [vp, ci, ci, ci, vp, vp, vp]
    L.wpa_mask_counts.argtypes = [ci, ci, ci, vp, vp]
    L.wpa_kv_write_i8.argtypes = [vp, vp, ci, ci, ci, vp, ci, vp, vp, vp, vp, vp]
    L.wpa_prefill_attn_i8_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_mask_counts_chunk.argtypes = [ci, ci, ci, ci, vp, vp]
    L.wpa_prefill_attn_fused_q.argtypes = [vp, ci, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    L.wpa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    L.wpa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.wpa_decode_attn_i8.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, ci, vp, ci, ci, ci, ci, ci, cf, vp,
                                     ctypes.c_size_t, vp, ci, vp]
    L.wpa_status_string.argtypes = [ci]
    L.wpa_status_string.restype = ctypes.c_char_p
    return L


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for f in ("wpa_quantize_q_rows", "wpa_prefill_attn_i8", "wpa_mask_counts", "wpa_kv_write_i8",
              "wpa_prefill_attn_i8_chunk", "wpa_mask_counts_chunk", "wpa_decode_attn_i8",
              "wpa_decode_workspace_bytes", "wpa_prefill_attn_fused_q", "wpa_decode_attn_i8_noalloc",
              "wpa_status_string"):
        assert f in fns


def test_library_exports_every_declared_symbol(lib):
    for f in declared_functions():
        assert hasattr(lib, f), f


def test_status_strings(lib):
    assert lib.wpa_status_string(0) == b"WPA_OK"
    for s in (1, 2, 3, 4, 5):
        assert lib.wpa_status_string(s).startswith(b"WPA_ERR")
    assert lib.wpa_status_string(99) == b"unknown status"


# Fake, never-dereferenced, 256-aligned addresses: every call below must be
# rejected by host validation before the library touches the device.
P = ctypes.c_void_p(0x100000)


def attn(lib, **kw):
    args = dict(q=P, qs=P, k=P, v=P, ks=P, vs=P, pt=P, n_pool=4, n=64, hq=4, hkv=2, W=0, S=0,
                scale=0.0625, out=P, dtype=1)
    args.update(kw)
    return lib.wpa_prefill_attn_i8(args["q"], args["qs"], args["k"], args["v"], args["ks"], args["vs"],
                                   args["pt"], args["n_pool"], args["n"], args["hq"], args["hkv"],
                                   args["W"], args["S"], args["scale"], args["out"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), SHAPE),
    (dict(hq=0), SHAPE),
    (dict(hkv=0), SHAPE),
    (dict(hq=6, hkv=4), SHAPE),
    (dict(S=-1), SHAPE),
    (dict(scale=0.0), SHAPE),
    (dict(scale=-1.0), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(scale=float("nan")), SHAPE),
    (dict(n_pool=3), SHAPE),              # 64 tokens need 4 pages
    (dict(dtype=7), UNSUP),
    (dict(q=None), NULL),
    (dict(k=None), NULL),
    (dict(pt=None), NULL),
    (dict(out=None), NULL),
    (dict(vs=None), NULL),
    (dict(k=ctypes.c_void_p(0x100004)), UNSUP),   # pools must be 16-byte aligned
    (dict(q=ctypes.c_void_p(0x100008)), UNSUP),
])
def test_attention_rejects_invalid_arguments(lib, kw, status):
    assert attn(lib, **kw) == status


def test_attention_zero_tokens_is_a_noop(lib):
    assert attn(lib, n=0, q=None, k=None, out=None, n_pool=0) == OK


def test_quantize_rejects_invalid_arguments(lib):
    q = lib.wpa_quantize_q_rows
    assert q(P, 1, -1, 4, P, P, None) == SHAPE
    assert q(P, 1, 4, 0, P, P, None) == SHAPE
    assert q(P, 5, 4, 4, P, P, None) == UNSUP
    assert q(None, 1, 4, 4, P, P, None) == NULL
    assert q(P, 1, 4, 4, None, P, None) == NULL
    assert q(P, 1, 4, 4, P, None, None) == NULL
    assert q(ctypes.c_void_p(0x100002), 1, 4, 4, P, P, None) == UNSUP
    assert q(None, 1, 0, 4, None, None, None) == OK


def test_mask_counts_rejects_invalid_arguments(lib):
    m = lib.wpa_mask_counts
    assert m(-1, 0, 0, P, None) == SHAPE
    assert m(10, 4, -1, P, None) == SHAPE
    assert m(10, 4, 1, None, None) == NULL
    assert m(0, 4, 1, None, None) == OK


def test_kv_write_rejects_invalid_arguments(lib):
    def w(k=P, v=P, dtype=1, n=4, hkv=2, slots=P, pages=1, kp=P, vp=P, ks=P, vs=P):
        return lib.wpa_kv_write_i8(k, v, dtype, n, hkv, slots, pages, kp, vp, ks, vs, None)
    assert w(n=-1) == SHAPE
    assert w(hkv=0) == SHAPE
    assert w(pages=-1) == SHAPE
    assert w(dtype=3) == UNSUP
    for name in ("k", "v", "slots", "kp", "vp", "ks", "vs"):
        assert w(**{name: None}) == NULL, name
    assert w(k=ctypes.c_void_p(0x100004)) == UNSUP
    assert w(vp=ctypes.c_void_p(0x100008)) == UNSUP
    assert w(n=0, k=None, v=None, slots=None, kp=None, vp=None, ks=None, vs=None) == OK


def test_chunk_entry_points_reject_invalid_arguments(lib):
    def c(q_start=32, n=64, n_pool=6, **kw):
        args = dict(q=P, qs=P, k=P, v=P, ks=P, vs=P, pt=P, hq=4, hkv=2, W=0, S=0, scale=0.0625, out=P, dtype=1)
        args.update(kw)
        return lib.wpa_prefill_attn_i8_chunk(args["q"], args["qs"], args["k"], args["v"], args["ks"], args["vs"],
                                             args["pt"], n_pool, q_start, n, args["hq"], args["hkv"], args["W"],
                                             args["S"], args["scale"], args["out"], args["dtype"], None)
    assert c(q_start=-16) == SHAPE
    assert c(n_pool=5) == SHAPE            # keys 0..95 need 6 pages
    assert c(q_start=8) == UNSUP           # the chunk must start on a page
    assert c(q=None) == NULL
    assert c(n=0, q=None, out=None) == OK
    m = lib.wpa_mask_counts_chunk
    assert m(-16, 10, 4, 1, P, None) == SHAPE
    assert m(16, -1, 4, 1, P, None) == SHAPE
    assert m(16, 10, 4, 1, None, None) == NULL
    assert m(16, 0, 4, 1, None, None) == OK


def test_fused_q_rejects_invalid_arguments(lib):
    def f(q=P, q_dtype=1, q_start=0, n=64, n_pool=4, **kw):
        args = dict(k=P, v=P, ks=P, vs=P, pt=P, hq=4, hkv=2, W=0, S=0, scale=0.0625, out=P, dtype=1)
        args.update(kw)
        return lib.wpa_prefill_attn_fused_q(q, q_dtype, args["k"], args["v"], args["ks"], args["vs"], args["pt"],
                                            n_pool, q_start, n, args["hq"], args["hkv"], args["W"], args["S"],
                                            args["scale"], args["out"], args["dtype"], None)
    assert f(q_dtype=0) == UNSUP           # float32 Q goes through wpa_quantize_q_rows
    assert f(q_dtype=7) == UNSUP
    assert f(n=-1) == SHAPE
    assert f(hq=6, hkv=4) == SHAPE
    assert f(n_pool=3) == SHAPE
    assert f(q_start=-16) == SHAPE
    assert f(scale=float("nan")) == SHAPE
    assert f(q_start=8, n_pool=5) == UNSUP
    assert f(q=ctypes.c_void_p(0x100002)) == UNSUP
    assert f(dtype=5) == UNSUP
    assert f(q=None) == NULL
    assert f(out=None) == NULL
    assert f(pt=None) == NULL
    assert f(n=0, q=None, out=None) == OK


def test_decode_workspace_size(lib):
    ws = lib.wpa_decode_workspace_bytes
    # splits of 8 pages over the longest key list the tables allow: 260 floats per (sequence, head, split)
    assert ws(3, 8, 100, 0, 0) == 3 * 8 * 13 * 260 * 4       # full causal: 100 blocks -> 13 splits
    assert ws(3, 8, 2048, 256, 1) == 3 * 8 * 33 * 260 * 4    # window: 257 blocks -> 33 splits
    assert ws(3, 8, 5, 256, 1) == 3 * 8 * 1 * 260 * 4
    assert ws(0, 8, 5, 0, 0) == 0


def test_decode_rejects_invalid_arguments(lib):
    need = lib.wpa_decode_workspace_bytes(2, 8, 10, 4, 1)

    def d(q=P, n_pool=4, pt=P, max_blocks=10, lens=P, batch=2, hq=8, hkv=2, W=4, S=1, scale=0.0625, ws=P,
          ws_bytes=None, out=P, dtype=1):
        return lib.wpa_decode_attn_i8(q, P, P, P, P, P, n_pool, pt, max_blocks, lens, batch, hq, hkv, W, S, scale,
                                      ws, need if ws_bytes is None else ws_bytes, out, dtype, None)
    assert d(batch=-1) == SHAPE
    assert d(hq=6, hkv=4) == SHAPE
    assert d(max_blocks=0) == SHAPE
    assert d(n_pool=0) == SHAPE
    assert d(S=-1) == SHAPE
    assert d(scale=0.0) == SHAPE
    assert d(ws_bytes=need - 1) == SHAPE
    assert d(dtype=9) == UNSUP
    # 17 query heads per KV head are accepted (two groups of heads); batch 0 launches nothing
    assert d(hq=34, hkv=2, batch=0, q=None, lens=None, ws=None, out=None) == OK
    assert d(q=None) == NULL
    assert d(lens=None) == NULL
    assert d(ws=None) == NULL
    assert d(ws=ctypes.c_void_p(0x100004)) == UNSUP
    assert d(batch=0, q=None, lens=None, ws=None, out=None) == OK


def test_decode_noalloc_rejects_invalid_arguments(lib):
    """The no-allocation decode: the workspace checks are replaced by the fixed
    buffer's size limit, checked on the host before any HIP call."""
    TOO_LARGE = 5

    def d(q=P, n_pool=4, pt=P, max_blocks=10, lens=P, batch=2, hq=8, hkv=2, W=4, S=1, scale=0.0625, out=P,
          dtype=1):
        return lib.wpa_decode_attn_i8_noalloc(q, P, P, P, P, P, n_pool, pt, max_blocks, lens, batch, hq, hkv, W, S,
                                              scale, out, dtype, None)
    lib.wpa_decode_attn_i8_noalloc.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                                                        ctypes.c_void_p] + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.wpa_decode_attn_i8_noalloc.restype = ctypes.c_int
    assert d(batch=-1) == SHAPE
    assert d(hq=6, hkv=4) == SHAPE
    assert d(scale=float("nan")) == SHAPE
    assert d(dtype=9) == UNSUP
    assert d(hq=34, hkv=2, batch=0, q=None, lens=None, out=None) == OK
    assert d(q=None) == NULL
    assert d(out=None) == NULL
    assert d(batch=0, q=None, lens=None, out=None) == OK
    # one more sequence than the 64 MiB buffer holds (16 heads x 33 splits x 260 floats each)
    limit = 64 << 20
    per_seq = lib.wpa_decode_workspace_bytes(1, 16, 2048, 256, 1)
    fit = limit // per_seq
    assert d(batch=fit + 1, hq=16, hkv=4, max_blocks=2048, W=256, S=1) == TOO_LARGE
    assert lib.wpa_status_string(TOO_LARGE).startswith(b"WPA_ERR_TOO_LARGE")


def test_host_block_list_matches_oracle_counts():
    """The traversal the kernels use (csrc/wpa_common.h, tile_blocks) restated
    by reading its integer formulas from the header and evaluating them for
    every tile: it must give exactly the oracle's attended counts."""
    import numpy as np
    import oracle
    src = open(os.path.join(ROOT, "windowed_int8_paged_amd", "csrc", "wpa_common.h")).read()
    assert "tb.n_total = tb.n_sink + (n_blk_q - tb.win_start);" in src

    def tile_blocks(qt, W, S):
        n_blk_q = qt + 1
        if W <= 0:
            n_sink, win_start = 0, 0
        else:
            rsb = max(0, n_blk_q - W)
            win_start, n_sink = rsb, min(S, rsb)
        return n_sink + (n_blk_q - win_start)

    for (n, W, S) in [(1000, 8, 1), (333, 3, 5), (4096, 256, 1), (500, 0, 3), (257, 1, 0)]:
        counts = np.array([16 * (tile_blocks(t // 16, W, S) - 1) + t % 16 + 1 for t in range(n)])
        assert np.array_equal(counts, oracle.mask_counts(n, W, S))
