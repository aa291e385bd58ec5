"""GPU parity of the KV-pool writer through the C ABI (bit-exact codes and
scales against the oracle's writer; untouched pool rows keep their bytes).

The writer fills the pool the int8 tensor-core prefill attention page reads
("Why the attention, and why tensor cores": 16-token int8 pages, one scale per
token and KV head), quantizing each row with the page's per-row formula."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(k, v, slots, kp, vp, ks, vs, as_bf16=None):
    """k, v: float32 arrays, or uint16 bf16 bit patterns when as_bf16 is given."""
    import windowed_int8_paged_amd as wpa
    if as_bf16 is not None:
        kd = torch.from_numpy(as_bf16[0].view(np.int16)).cuda().view(torch.bfloat16)
        vd = torch.from_numpy(as_bf16[1].view(np.int16)).cuda().view(torch.bfloat16)
    else:
        kd, vd = _to_dev(k), _to_dev(v)
    d = [_to_dev(x) for x in (kp, vp, ks, vs)]
    wpa.kv_write_i8(kd, vd, _to_dev(slots.astype(np.int32)), *d)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in d]


def _same(got, want):
    for g, w in zip(got, want):
        assert g.dtype == w.dtype
        assert np.array_equal(g.view(np.uint8) if g.dtype == np.int8 else g.view(np.uint32),
                              w.view(np.uint8) if w.dtype == np.int8 else w.view(np.uint32))


@pytest.mark.parametrize("n,hkv,pages,seed", [(37, 2, 4, 1), (1, 1, 1, 2), (200, 4, 16, 3), (1000, 8, 70, 4)])
def test_kv_write_bit_exact(n, hkv, pages, seed):
    kb, vb, k, v, slots, kp, vp, ks, vs = workloads.make_kv_rows(n, hkv, pages, seed)
    want = oracle.kv_write_i8(k, v, slots, kp, vp, ks, vs)
    print(f"kv_write n={n} hkv={hkv} pages={pages} seed={seed}", flush=True)
    _same(_run(k, v, slots, kp, vp, ks, vs, as_bf16=(kb, vb)), want)  # bf16 container
    _same(_run(k, v, slots, kp, vp, ks, vs), want)                      # f32 container


def test_kv_write_full_float32_values_and_zero_rows():
    kb, vb, k, v, slots, kp, vp, ks, vs = workloads.make_kv_rows(300, 4, 20, seed=8)
    rng = np.random.default_rng(80)
    k = rng.standard_normal(k.shape).astype(np.float32) * np.float32(3.7)  # not on the bf16 grid
    v = rng.standard_normal(v.shape).astype(np.float32) * np.float32(1e-3)
    k[5] = 0.0
    v[7, 2] = 0.0
    print("kv_write float32 values", flush=True)
    _same(_run(k, v, slots, kp, vp, ks, vs), oracle.kv_write_i8(k, v, slots, kp, vp, ks, vs))


def test_kv_write_skips_slots_outside_the_pool():
    kb, vb, k, v, slots, kp, vp, ks, vs = workloads.make_kv_rows(40, 2, 4, seed=12)
    slots = slots.copy()
    slots[[0, 9, 33]] = [-1, 64, 2**30]  # 64 = 16 * n_pool_pages is one past the end
    print("kv_write out-of-range slots", flush=True)
    want = oracle.kv_write_i8(k, v, slots, kp, vp, ks, vs)
    _same(_run(k, v, slots, kp, vp, ks, vs, as_bf16=(kb, vb)), want)


def test_kv_write_32k_shape():
    # the 32k workload's whole K/V write: 32768 tokens x 4 KV heads into a 2048-page pool
    kb, vb, k, v, slots, kp, vp, ks, vs = workloads.make_kv_rows(32768, 4, 2048, seed=1003)
    print("kv_write 32k shape", flush=True)
    _same(_run(k, v, slots, kp, vp, ks, vs, as_bf16=(kb, vb)), oracle.kv_write_i8(k, v, slots, kp, vp, ks, vs))


def test_kv_write_zero_tokens_is_a_noop():
    import windowed_int8_paged_amd as wpa
    kp = torch.zeros((1, 16, 1, 256), dtype=torch.int8, device="cuda")
    sc = torch.zeros((1, 16, 1), dtype=torch.float32, device="cuda")
    e = torch.empty((0, 1, 256), dtype=torch.bfloat16, device="cuda")
    wpa.kv_write_i8(e, e, torch.empty((0,), dtype=torch.int32, device="cuda"), kp, kp.clone(), sc, sc.clone())
    torch.cuda.synchronize()
    assert int(kp.abs().sum()) == 0
