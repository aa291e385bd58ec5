"""Seeded random shapes through every prefill entry point (C ABI), and seeded random
decode batches, each checked against the oracle at the acceptance bars.

The prefill shapes are drawn from fixed seeds (16 from one, 60 from another): lengths from 1 to 1500 tokens
(ragged tails included), 1 to 8 query heads per KV head, 1 to 4 KV heads,
window and sink blocks covering full causal, narrow and over-wide windows,
and a chunk start on a random page boundary.  For each shape the int8-Q path,
the fused-Q path and the chunked path must agree bitwise on the rows they
share, and the int8-Q output must meet the oracle bars (int8 tensor-core
prefill attention page, "Why the attention, and why tensor cores")."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import check_parity, upload

pytestmark = pytest.mark.gpu


def _shapes(n_cases=16, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        hkv = int(rng.integers(1, 5))
        g = int(rng.integers(1, 9))
        n = int(rng.integers(1, 1501))
        kind = rng.integers(0, 3)
        if kind == 0:
            w, s = 0, int(rng.integers(0, 3))          # full causal (sink ignored)
        elif kind == 1:
            w, s = int(rng.integers(1, 6)), int(rng.integers(0, 4))
        else:
            w, s = int(rng.integers(60, 200)), 1       # window wider than most sequences
        q_start = 16 * int(rng.integers(0, (n + 15) // 16))
        out.append((n, g * hkv, hkv, w, s, q_start, int(rng.integers(0, 2**31))))
    return out


@pytest.mark.parametrize("n,hq,hkv,W,S,q_start,seed", _shapes() + _shapes(60, 777))
def test_random_shape(n, hq, hkv, W, S, q_start, seed):
    import windowed_int8_paged_amd as wpa
    case = workloads.make_case(n_tokens=n, n_q_heads=hq, n_kv_heads=hkv, window_blocks=W, sink_blocks=S,
                               seed=seed, extra_pool_frac=0.25)
    dev = upload(case)
    print(f"random shape n={n} hq={hq} hkv={hkv} W={W} S={S} q_start={q_start}", flush=True)
    q_i8, q_scale = wpa.quantize_q_rows(dev["q_bf16"])
    args = (dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"], dev["page_table"], W, S,
            case.softmax_scale)
    full = wpa.prefill_attn_i8(q_i8, q_scale, *args, out_dtype=torch.float32)
    fused = wpa.prefill_attn_fused_q(dev["q_bf16"], *args, out_dtype=torch.float32)
    q_c = dev["q_bf16"][q_start:].contiguous()
    qi_c, qs_c = wpa.quantize_q_rows(q_c)
    chunk = wpa.prefill_attn_i8_chunk(q_start, qi_c, qs_c, *args, out_dtype=torch.float32)
    counts = wpa.mask_counts_chunk(q_start, n - q_start, W, S)
    torch.cuda.synchronize()
    assert torch.equal(fused, full)
    assert torch.equal(chunk, full[q_start:])
    assert np.array_equal(counts.cpu().numpy(), oracle.mask_counts(n, W, S)[q_start:])
    # the oracle on at most 6 tiles: first, last, the chunk's first and three more
    nt = (n + 15) // 16
    rng = np.random.default_rng(seed)
    tiles = sorted({0, nt - 1, q_start // 16, *rng.integers(0, nt, size=3).tolist()})
    check_parity(case, full, tiles=tiles, label=f"random n={n}")


def _decode_batches(n_cases=40, seed=778):
    """Ragged batches of 1-4 sequences of 1-3000 tokens, 1-20 query heads per KV head,
    1-4 KV heads, full causal or a 1-23-block window, 0-3 sink blocks."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        hkv = int(rng.integers(1, 5))
        g = int(rng.integers(1, 21))
        lens = sorted(int(x) for x in rng.integers(1, 3001, size=int(rng.integers(1, 5))))
        w = int(rng.choice([0, int(rng.integers(1, 24))]))
        s = int(rng.integers(0, 4))
        out.append((lens, g * hkv, hkv, w, s, int(rng.integers(0, 2**31))))
    return out


@pytest.mark.parametrize("lens,hq,hkv,W,S,seed", _decode_batches())
def test_random_decode_batch(lens, hq, hkv, W, S, seed):
    """Every sequence's row against the prefill oracle's row t (bf16 output equal to the RNE
    of the fp32 one); unattended blocks point at the NaN-scaled page 0."""
    from gpu_util import poison_unattended_blocks
    from test_gpu_decode import check_batch, run_decode, upload_batch
    d = poison_unattended_blocks(workloads.make_decode_batch(lens, hq, hkv, W, S, seed=seed))
    dev = upload_batch(d)
    print(f"random decode lens={lens} hq={hq} hkv={hkv} W={W} S={S}", flush=True)
    o32 = run_decode(d, dev, torch.float32)
    check_batch(d, o32, f"random decode {lens}")
    o16 = run_decode(d, dev, torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16))
