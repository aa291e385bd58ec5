"""GPU parity of the split-KV decode (wpa_decode_attn_i8) through the C ABI.

Each sequence's new token is its last position t = seq_len - 1, attending
A(t) under the prefill path's mask with the same int8 scheme (int8
tensor-core prefill attention page, "Why the attention, and why tensor
cores").  The oracle is therefore the prefill oracle's row t of that sequence
(workloads.decode_row_case), checked at the same acceptance bars.  Every
block a query does not attend points at the pool's NaN-scaled page 0, so a
stray read shows as a non-finite output."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import check_parity, poison_unattended_blocks

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def upload_batch(d):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = torch.from_numpy(d.q_bf16.view(np.int16)).cuda().view(torch.bfloat16)
    return dict(q=q, k_pool=t(d.k_pool), v_pool=t(d.v_pool), k_scale=t(d.k_scale), v_scale=t(d.v_scale),
                tables=t(d.page_tables), lens=t(d.seq_lens))


def run_decode(d, dev, out_dtype=torch.bfloat16, workspace=None):
    import windowed_int8_paged_amd as wpa
    q_i8, q_scale = wpa.quantize_q_rows(dev["q"])
    out = wpa.decode_attn_i8(q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                             dev["tables"], dev["lens"], d.window_blocks, d.sink_blocks, d.softmax_scale,
                             out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return out


def check_batch(d, out, label, seqs=None):
    res = []
    for b in (range(len(d.seq_lens)) if seqs is None else seqs):
        L = int(d.seq_lens[b])
        case = workloads.decode_row_case(d, b)
        full = torch.full((L, d.n_q_heads, 256), float("nan"), dtype=out.dtype)
        full[L - 1] = out[b].cpu()
        res.append(check_parity(case, full, tiles=[(L - 1) // 16], rows=[L - 1], label=f"{label} seq {b} len {L}"))
    return res


@pytest.mark.parametrize("lens,hq,hkv,W,S,seed", [
    ([1, 15, 16, 17, 130, 700, 2000], 8, 2, 8, 1, 51),   # windowed: 9-block lists, two splits
    ([5, 300, 1500], 4, 1, 0, 0, 52),                     # full causal: up to 94 blocks, 12 splits
    ([40, 1000], 16, 1, 4, 2, 53),                         # 16 query heads per KV head
    ([33, 257], 4, 4, 3, 0, 54),                           # one query head per KV head
    ([90, 600], 6, 2, 5, 1, 56),                           # 3 heads: a partly filled (head, page) row tile
    ([129, 520], 16, 2, 6, 0, 57),                         # 8 heads: two row tiles of the PV operand
    ([64, 400], 10, 2, 0, 0, 58),                          # 5 heads: two row tiles, the second with one head
    ([50, 700], 32, 1, 4, 1, 59),                          # 32 query heads per KV head: two groups of 16
    ([90, 400], 40, 2, 3, 0, 60),                          # 20 per KV head: a group of 16 and one of 4
])
def test_decode_parity(lens, hq, hkv, W, S, seed):
    d = poison_unattended_blocks(workloads.make_decode_batch(lens, hq, hkv, W, S, seed=seed))
    dev = upload_batch(d)
    _say(f"decode lens={lens} hq={hq} hkv={hkv} W={W} S={S}")
    o32 = run_decode(d, dev, torch.float32)
    r = check_batch(d, o32, "f32")
    _say(f"  worst rel {max(x['rel_mirror'] for x in r):.2e}, frob {max(x['frob_exact'] for x in r):.2e}")
    o16 = run_decode(d, dev, torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_decode_zero_and_clamped_lengths():
    d = poison_unattended_blocks(workloads.make_decode_batch([200, 100], 8, 2, 4, 1, seed=55, max_blocks=13))
    dev = upload_batch(d)
    lens = torch.tensor([0, 100000], dtype=torch.int32, device="cuda")  # 0 -> zero row; above the table -> 208
    dev["lens"] = lens
    _say("decode zero and clamped lengths")
    out = run_decode(d, dev, torch.float32)
    assert torch.all(out[0] == 0)
    d.seq_lens = np.array([1, 13 * 16], dtype=np.int32)
    d.page_tables[1] = np.random.default_rng(0).permutation(d.k_pool.shape[0] - 1)[:13] + 1
    poison_unattended_blocks(d)
    dev = upload_batch(d)
    dev["lens"] = lens
    out = run_decode(d, dev, torch.float32)
    check_batch(d, out, "clamped", seqs=[1])


def test_decode_reused_workspace_and_determinism():
    import windowed_int8_paged_amd as wpa
    d = poison_unattended_blocks(workloads.make_decode_batch([77, 900, 3000], 8, 2, 16, 1, seed=56))
    dev = upload_batch(d)
    need = wpa.decode_workspace_bytes(3, 8, d.page_tables.shape[1], 16, 1)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-patterned scratch
    _say("decode reused workspace")
    a = run_decode(d, dev, torch.float32, workspace=ws)
    b = run_decode(d, dev, torch.float32, workspace=ws)
    assert torch.equal(a, b)
    check_batch(d, a, "ws")


def test_decode_32k_shape_sampled():
    """The bench shape: every sequence at 32768 tokens, 16 / 4 heads, window 256
    blocks + 1 sink, every block on a page of its own, the unattended ones then
    pointed at the poisoned page; two sequences checked."""
    d = poison_unattended_blocks(workloads.make_decode_batch([32768] * 8, 16, 4, 256, 1, seed=57, owned_pages=True))
    dev = upload_batch(d)
    _say("decode 32k shape")
    out = run_decode(d, dev, torch.bfloat16)
    check_batch(d, out, "32k", seqs=[0, 5])
