"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer work is bit-exact (Q codes and scales, attended counts); the attention
output is within max|d| <= 2e-3*max|O| of the int8 mirror (fp32 outputs with
no further allowance) and within 3e-2 relative Frobenius of exact attention.
bf16 outputs are additionally allowed half a bf16 ulp (their own rounding),
and must equal the round-to-nearest-even of the same kernel's fp32 output bit
for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import check_parity, oracle_rows, run, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import windowed_int8_paged_amd  # noqa: F401  (fails loudly if the library is missing)


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- Q codes

@pytest.mark.parametrize("container", ["bf16", "f32"])
def test_quantize_q_rows_bit_exact(container):
    import windowed_int8_paged_amd as wpa
    rng = np.random.default_rng(77)
    case = workloads.make_case(n_tokens=333, n_q_heads=6, n_kv_heads=2, window_blocks=0,
                               sink_blocks=0, seed=5, q_outlier_frac=0.05)
    q = case.q_f32.copy()
    q[3, 1] = 0.0                                        # zero row
    q[4, 2] = (np.arange(256) % 9 - 4).astype(np.float32) / 8 * (127 / 4)  # exact halves
    q[5, 0, :7] = np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 127.0], dtype=np.float32) / 8
    q[5, 0, 7:] = 0
    bits = workloads._round_to_bf16_bits(q)
    qf = workloads._bf16_bits_to_f32(bits)
    codes, scale = oracle.quantize_q_rows(qf)
    if container == "bf16":
        dq = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        dq = torch.from_numpy(qf).cuda()
    q_i8, q_scale = wpa.quantize_q_rows(dq)
    torch.cuda.synchronize()
    assert np.array_equal(q_i8.cpu().numpy(), codes)
    assert np.array_equal(q_scale.cpu().numpy().view(np.uint32), scale.view(np.uint32))
    del rng


# ---------------------------------------------------------------- mask counts

@pytest.mark.parametrize("n,W,S", [(64, 0, 0), (1000, 8, 1), (4096, 256, 1), (777, 3, 5),
                                   (17, 1, 0), (5000, 2, 0), (16384, 0, 0), (333, -4, 2)])
def test_mask_counts_bit_exact(n, W, S):
    import windowed_int8_paged_amd as wpa
    got = wpa.mask_counts(n, W, S).cpu().numpy()
    assert np.array_equal(got, oracle.mask_counts(n, W, S))


@pytest.mark.parametrize("name,total", [("32k", 126074880), ("64k", 260571136)])
def test_mask_counts_full_size(name, total):
    import windowed_int8_paged_amd as wpa
    cfg = workloads.CONFIGS[name]
    n, W, S = cfg["n_tokens"], cfg["window_blocks"], cfg["sink_blocks"]
    got = wpa.mask_counts(n, W, S).cpu().numpy()
    assert int(got.astype(np.int64).sum()) == total
    assert got.max() == 4112
    for tile in (0, 1, 255, 256, 257, n // 32, n // 16 - 1):
        rows = oracle.tile_rows(n, tile)
        keys = np.arange(0, rows[-1] + 1)
        assert np.array_equal(got[rows], oracle.attended_mask(rows, keys, W, S).sum(axis=1))


# ---------------------------------------------------------------- small cases, all rows

SMALL = [
    # n, hq, hkv, W, S, seed
    (64, 2, 1, 0, 0, 1),        # tiny-like, full causal
    (100, 4, 4, 2, 1, 2),       # MHA, ragged tail
    (1000, 8, 2, 8, 1, 3),      # GQA-4, windowed, ragged
    (777, 6, 2, 3, 0, 4),       # GQA-3 (odd: four query tiles per workgroup), no sink
    (515, 16, 2, 4, 2, 5),      # GQA-8 (4 waves per workgroup)
    (300, 2, 2, 1, 0, 6),       # window of one block
    (90, 4, 1, 1, 5, 7),        # sink larger than the window start
    (33, 4, 2, 300, 1, 8),      # window wider than the sequence
    (1, 4, 2, 0, 0, 9),         # a single token
    (16, 8, 2, 1, 1, 10),       # exactly one tile
]


@pytest.mark.parametrize("n,hq,hkv,W,S,seed", SMALL)
def test_small_parity(n, hq, hkv, W, S, seed):
    case = workloads.make_case(n_tokens=n, n_q_heads=hq, n_kv_heads=hkv, window_blocks=W,
                               sink_blocks=S, seed=seed, extra_pool_frac=0.3)
    dev = upload(case)
    _say(f"small case n={n} hq={hq} hkv={hkv} W={W} S={S}")
    _, _, o32 = run(case, dev, out_dtype=torch.float32)
    check_parity(case, o32, label="f32")
    _, _, o16 = run(case, dev, out_dtype=torch.bfloat16)
    check_parity(case, o16, label="bf16")
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_outlier_rows_small():
    """Outlier Q rows and saturated K tokens with log-uniform scales, full causal."""
    case = workloads.make_case(n_tokens=1500, n_q_heads=8, n_kv_heads=2, window_blocks=0,
                               sink_blocks=0, seed=11, scale_lo=1e-3, scale_hi=5e-2,
                               log_uniform_scales=True, q_outlier_frac=0.01, k_saturated_frac=0.02)
    _, _, o32 = run(case, out_dtype=torch.float32)
    check_parity(case, o32, label="outliers f32")


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_peaked_scores(scale):
    """Strongly peaked softmax rows: a softmax scale 16 and 64 times the
    default over outlier Q rows (channels x30) and saturated K tokens, so that
    a few keys carry nearly all of a row's weight and the reference rises by
    many bits at once.  The kernel is held to the int8 mirror's bar; the
    method itself (the mirror) is 9% (relative Frobenius) from exact attention
    on these rows, past the 3e-2 stated for the five workloads, so that
    comparison is reported, not asserted."""
    case = workloads.make_case(n_tokens=700, n_q_heads=8, n_kv_heads=2, window_blocks=6, sink_blocks=1,
                               seed=14, softmax_scale=scale, q_outlier_frac=0.2, k_saturated_frac=0.05,
                               out_dtype="f32")
    _say(f"peaked scores, softmax scale {scale}")
    _, _, o32 = run(case, out_dtype=torch.float32)
    r = check_parity(case, o32, label=f"peaked x{scale}", frob_bar=None)
    _say(f"peaked {scale}: {r}")


def test_tiny_config_both_containers():
    case = workloads.make_config("tiny")
    dev = upload(case)
    _, _, a = run(case, dev, q_key="q_bf16", out_dtype=torch.float32)
    _, _, b = run(case, dev, q_key="q_f32", out_dtype=torch.float32)
    assert torch.equal(a, b)
    r = check_parity(case, a, label="tiny")
    _say(f"tiny parity {r}")


def test_deterministic_and_stray_page_safe():
    """Run twice bitwise equal; unused pool pages carry NaN scales and random
    codes, so any read of them would make the output non-finite."""
    case = workloads.make_case(n_tokens=700, n_q_heads=8, n_kv_heads=2, window_blocks=4,
                               sink_blocks=1, seed=12, extra_pool_frac=1.0)
    dev = upload(case)
    _, _, a = run(case, dev)
    _, _, b = run(case, dev)
    assert torch.equal(a, b)
    assert torch.isfinite(a.float()).all()


def test_out_of_pool_page_ids_are_clamped():
    """Page-table entries outside the pool (negative, past the end) are clamped
    into it on the device, below 0 to page 0 and past the end to the last page:
    the output is the oracle's for the clamped table, and nothing outside the
    pool is read.  The sink block and two window blocks carry bad entries."""
    import dataclasses
    case = workloads.make_case(n_tokens=600, n_q_heads=8, n_kv_heads=2, window_blocks=5, sink_blocks=1, seed=13,
                               extra_pool_frac=0.3, poison_unused=False)
    n_pool = case.k_pool.shape[0]
    bad = case.page_table.copy()
    bad[0], bad[3], bad[20] = 2**31 - 1, -7, n_pool + 1000
    dev = upload(case)
    dev["page_table"] = torch.from_numpy(bad).cuda()
    _say("out-of-pool page ids")
    _, _, out = run(case, dev, out_dtype=torch.float32)
    clamped = dataclasses.replace(case, page_table=np.clip(bad, 0, n_pool - 1).astype(np.int32))
    check_parity(clamped, out, label="clamped page ids")


# ---------------------------------------------------------------- the five workloads, sampled

def sample_tiles(name, n_tokens, window_blocks, count=32):
    """The first and last tiles, the middle, the tiles around the window's
    fill-up, then seeded random tiles up to `count`."""
    nt = (n_tokens + 15) // 16
    tiles = {0, 1, 2, nt // 3, nt // 2, nt - 2, nt - 1}
    if window_blocks > 0:
        tiles |= {window_blocks - 1, window_blocks, window_blocks + 1}
    tiles = {t for t in tiles if 0 <= t < nt}
    rng = np.random.default_rng(sum(map(ord, name)))
    while len(tiles) < min(count, nt):
        tiles.add(int(rng.integers(0, nt)))
    return sorted(tiles)


@pytest.mark.parametrize("name", ["4k", "32k", "64k", "16k_full", "32k_gqa2", "32k_mha"])
def test_config_sampled_parity(name):
    """32 tiles per workload (fixed and random ones), in the benchmarked launch
    (bf16 Q quantized inside the attention, bf16 output), in the separate-quantize
    launch with bf16 and fp32 output; fp32 meets the plain bar."""
    import windowed_int8_paged_amd as wpa
    case = workloads.make_config(name)
    dev = upload(case)
    tiles = sample_tiles(name, case.n_tokens, case.window_blocks)
    _say(f"config {name}: {len(tiles)} tiles {tiles}")
    _, _, o16 = run(case, dev, out_dtype=torch.bfloat16)
    _, _, o32 = run(case, dev, out_dtype=torch.float32)
    fused = wpa.prefill_attn_fused_q(dev["q_bf16"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                     dev["page_table"], case.window_blocks, case.sink_blocks, case.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(fused, o16)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.isfinite(o16.float()).all()
    ref = oracle_rows(case, tiles)
    r32 = check_parity(case, o32, tiles=tiles, label=f"{name} f32", ref=ref)
    r16 = check_parity(case, o16, tiles=tiles, label=f"{name} bf16", ref=ref)
    _say(f"config {name}: f32 {r32} bf16 {r16}")
