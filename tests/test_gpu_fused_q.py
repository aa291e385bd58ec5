"""GPU parity of the fused-Q attention (wpa_prefill_attn_fused_q) through the C ABI.

The entry point takes bf16 Q and quantizes each query row inside the
attention kernel with the per-row formula of the int8 tensor-core prefill
attention page ("Why the attention, and why tensor cores": one scale per
row).  Its output must be bitwise that of the separate quantize launch
followed by the int8-Q attention, and within the acceptance bars of the
oracle on its own."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_parity, upload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def separate(case, dev, out_dtype, q_start=0, n=None):
    import windowed_int8_paged_amd as wpa
    n = case.n_tokens - q_start if n is None else n
    q = dev["q_bf16"][q_start:q_start + n].contiguous()
    q_i8, q_scale = wpa.quantize_q_rows(q)
    out = wpa.prefill_attn_i8_chunk(q_start, q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                    dev["v_scale"], dev["page_table"], case.window_blocks, case.sink_blocks,
                                    case.softmax_scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def fused(case, dev, out_dtype, q_start=0, n=None):
    import windowed_int8_paged_amd as wpa
    n = case.n_tokens - q_start if n is None else n
    q = dev["q_bf16"][q_start:q_start + n].contiguous()
    out = wpa.prefill_attn_fused_q(q, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                   dev["page_table"], case.window_blocks, case.sink_blocks, case.softmax_scale,
                                   out_dtype=out_dtype, q_start=q_start)
    torch.cuda.synchronize()
    return out


CASES = [
    # n, hq, hkv, W, S, seed
    (64, 2, 1, 0, 0, 41),       # GQA-2: two query tiles per workgroup
    (1000, 8, 2, 8, 1, 42),     # GQA-4, windowed, ragged tail
    (777, 6, 2, 3, 0, 43),      # GQA-3: four query tiles per workgroup
    (515, 16, 2, 4, 2, 44),     # GQA-8
    (33, 4, 4, 300, 1, 45),     # MHA, window wider than the sequence
    (1, 4, 2, 0, 0, 46),        # a single token
]


@pytest.mark.parametrize("n,hq,hkv,W,S,seed", CASES)
def test_fused_equals_separate_and_oracle(n, hq, hkv, W, S, seed):
    case = workloads.make_case(n_tokens=n, n_q_heads=hq, n_kv_heads=hkv, window_blocks=W, sink_blocks=S,
                               seed=seed, extra_pool_frac=0.3)
    dev = upload(case)
    _say(f"fused q n={n} hq={hq} hkv={hkv} W={W} S={S}")
    for dt in (torch.float32, torch.bfloat16):
        a = fused(case, dev, dt)
        assert torch.equal(a, separate(case, dev, dt))
    check_parity(case, a, label="fused bf16")


def test_fused_outlier_rows():
    """Rows with a few channels x30: the row scale is set by the outliers."""
    case = workloads.make_case(n_tokens=700, n_q_heads=8, n_kv_heads=2, window_blocks=0, sink_blocks=0, seed=47,
                               scale_lo=1e-3, scale_hi=5e-2, log_uniform_scales=True, q_outlier_frac=0.02,
                               k_saturated_frac=0.02)
    dev = upload(case)
    a = fused(case, dev, torch.float32)
    assert torch.equal(a, separate(case, dev, torch.float32))
    check_parity(case, a, label="fused outliers")


def test_fused_zero_rows():
    """A Q row of zeros has scale 0 and codes 0: its scores are all 0 and it
    averages V over its keys, as in the separate path."""
    case = workloads.make_case(n_tokens=200, n_q_heads=4, n_kv_heads=2, window_blocks=3, sink_blocks=1, seed=48,
                               extra_pool_frac=0.2)
    dev = upload(case)
    dev["q_bf16"][5] = 0
    dev["q_bf16"][150, 2] = 0
    a = fused(case, dev, torch.float32)
    assert torch.equal(a, separate(case, dev, torch.float32))
    assert torch.isfinite(a).all()


@pytest.mark.parametrize("q_start,n", [(320, 180), (160, 192), (0, 96)])
def test_fused_chunk(q_start, n):
    case = workloads.make_case(n_tokens=500, n_q_heads=8, n_kv_heads=2, window_blocks=4, sink_blocks=2, seed=49,
                               extra_pool_frac=0.3)
    dev = upload(case)
    _say(f"fused chunk q_start={q_start} n={n}")
    a = fused(case, dev, torch.bfloat16, q_start, n)
    assert torch.equal(a, separate(case, dev, torch.bfloat16, q_start, n))


def test_fused_32k_equals_separate():
    """The benchmarked workload: whole output bitwise equal to the separate path."""
    case = workloads.make_config("32k")
    dev = upload(case)
    _say("fused q 32k")
    a = fused(case, dev, torch.bfloat16)
    b = separate(case, dev, torch.bfloat16)
    assert torch.equal(a, b)
    assert torch.isfinite(a.float()).all()
