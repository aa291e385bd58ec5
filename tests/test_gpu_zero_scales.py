"""GPU parity with zero and tiny V scales (prefill and decode, through the C ABI).

The KV writer stores scale 0 for an all-zero row (one scale per token: amax 0
gives scale 0 and codes 0, as for the per-row Q scale of the int8
tensor-core prefill attention page, "Why the attention, and why tensor
cores").  Such keys still count in the softmax denominator l while adding
nothing to P*V, so a row whose first keys all have zero V must come out as
the oracle says, not as NaN.  Keys whose V scale is tiny but not zero make
the running per-row reference jump by tens of bits when ordinary keys follow;
the oracle fixes the result there too."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_parity, upload
from test_gpu_decode import check_batch, run_decode, upload_batch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _zero_v(case, tokens):
    pages = case.page_table[tokens // 16]
    slots = tokens % 16
    case.v_pool[pages, slots] = 0
    case.v_scale[pages, slots] = 0.0


def _prefill(case, dev, dt):
    import windowed_int8_paged_amd as wpa
    q_i8, q_scale = wpa.quantize_q_rows(dev["q_bf16"])
    out = wpa.prefill_attn_i8(q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                              dev["page_table"], case.window_blocks, case.sink_blocks, case.softmax_scale,
                              out_dtype=dt)
    fused = wpa.prefill_attn_fused_q(dev["q_bf16"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                     dev["page_table"], case.window_blocks, case.sink_blocks, case.softmax_scale,
                                     out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(out, fused)
    return out


@pytest.mark.parametrize("W,S", [(0, 0), (6, 1)])
def test_prefill_leading_zero_v(W, S):
    """V of the first 320 tokens is zero: those rows give exactly 0; later rows
    see only zero-scale keys in their first steps."""
    case = workloads.make_case(n_tokens=700, n_q_heads=8, n_kv_heads=2, window_blocks=W, sink_blocks=S, seed=61,
                               extra_pool_frac=0.2)
    _zero_v(case, np.arange(320))
    dev = upload(case)
    _say(f"prefill leading zero V W={W} S={S}")
    out = _prefill(case, dev, torch.float32)
    assert torch.all(out[:320] == 0)
    check_parity(case, out, label="leading zero V")


def test_prefill_scattered_zero_v():
    """A fifth of the tokens, and the whole sink block, have zero V."""
    case = workloads.make_case(n_tokens=900, n_q_heads=16, n_kv_heads=4, window_blocks=5, sink_blocks=1, seed=62,
                               extra_pool_frac=0.2)
    rng = np.random.default_rng(62)
    tokens = np.union1d(np.arange(16), np.flatnonzero(rng.random(900) < 0.2))
    _zero_v(case, tokens)
    dev = upload(case)
    _say("prefill scattered zero V")
    check_parity(case, _prefill(case, dev, torch.bfloat16), label="scattered zero V")


def test_prefill_tiny_leading_v_scales():
    """V scales of the first 160 tokens times 2^-50: the reference of every
    later row rises by about 50 bits when ordinary keys arrive."""
    case = workloads.make_case(n_tokens=600, n_q_heads=8, n_kv_heads=2, window_blocks=0, sink_blocks=0, seed=63,
                               extra_pool_frac=0.2)
    tokens = np.arange(160)
    pages, slots = case.page_table[tokens // 16], tokens % 16
    case.v_scale[pages, slots] *= np.float32(2.0 ** -50)
    dev = upload(case)
    _say("prefill tiny leading V scales")
    out = _prefill(case, dev, torch.float32)
    check_parity(case, out, label="tiny V scales")


def test_decode_zero_v_splits():
    """Whole 8-page splits of zero V (sequence 1's first 800 tokens) and a
    sequence whose every key has zero V (exact zero row)."""
    d = workloads.make_decode_batch([300, 1500, 200], 8, 2, 0, 0, seed=64, owned_pages=True)
    for b, n in ((1, 800), (2, 200)):
        pages = d.page_tables[b, :(n + 15) // 16]
        d.v_pool[pages] = 0
        d.v_scale[pages] = 0.0
    dev = upload_batch(d)
    _say("decode zero V splits")
    out = run_decode(d, dev, torch.float32)
    assert torch.all(out[2] == 0)
    check_batch(d, out, "zero V", seqs=[0, 1])
