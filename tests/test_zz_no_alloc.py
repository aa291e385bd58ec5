"""The no-allocation decode entry point (wpa_decode_attn_i8_noalloc) through
the C ABI against the workspace entry point (wpa_decode_attn_i8): the same
kernels, so the outputs must be equal bit for bit, on two calls in a row, the
second with a smaller input (the fixed buffer keeps the first call's rows)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import poison_unattended_blocks
from test_gpu_decode import upload_batch

pytestmark = pytest.mark.gpu


def _both(d, out_dtype):
    import windowed_int8_paged_amd as wpa
    dev = upload_batch(d)
    q_i8, q_scale = wpa.quantize_q_rows(dev["q"])
    args = (q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"], dev["tables"], dev["lens"],
            d.window_blocks, d.sink_blocks, d.softmax_scale)
    ref = wpa.decode_attn_i8(*args, out_dtype=out_dtype)
    got = wpa.decode_attn_i8_noalloc(*args, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_decode_matches_workspace_decode():
    big = poison_unattended_blocks(workloads.make_decode_batch([4000, 33, 2100, 700], 16, 4, 8, 1, seed=91))
    print("no-alloc decode: 4 sequences, 16/4 heads, window 8 + 1 sink", flush=True)
    ref, got = _both(big, torch.float32)
    assert torch.isfinite(got).all()
    assert torch.equal(ref, got)
    small = poison_unattended_blocks(workloads.make_decode_batch([300, 17], 8, 2, 0, 0, seed=92))
    print("no-alloc decode: 2 shorter sequences, 8/2 heads, full causal", flush=True)
    ref, got = _both(small, torch.bfloat16)
    assert torch.isfinite(got.float()).all()
    assert torch.equal(ref, got)
