"""Helpers for the GPU parity tests: upload a seeded case, run the library
through its C ABI, and compare with the oracle at the stated tolerances."""
import numpy as np
import torch

import oracle
import workloads

# Acceptance bars: against the int8 mirror, max|d| <= 2e-3 * max|O|; against
# the exact attention, relative Frobenius error <= 3e-2.
TOL_MIRROR = 2e-3
TOL_EXACT_FROB = 3e-2


def upload(case, device="cuda"):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    q_bf16 = torch.from_numpy(case.q_bf16.view(np.int16)).to(device).view(torch.bfloat16)
    return dict(
        q_bf16=q_bf16,
        q_f32=t(case.q_f32),
        k_pool=t(case.k_pool), v_pool=t(case.v_pool),
        k_scale=t(case.k_scale), v_scale=t(case.v_scale),
        page_table=t(case.page_table),
    )


def run(case, dev=None, q_key="q_bf16", out_dtype=torch.bfloat16):
    import windowed_int8_paged_amd as wpa
    if dev is None:
        dev = upload(case)
    q_i8, q_scale = wpa.quantize_q_rows(dev[q_key])
    out = wpa.prefill_attn_i8(q_i8, q_scale, dev["k_pool"], dev["v_pool"], dev["k_scale"],
                              dev["v_scale"], dev["page_table"], case.window_blocks,
                              case.sink_blocks, case.softmax_scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return q_i8, q_scale, out


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 1e-30)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def rows_of_tiles(n_tokens, tiles):
    return np.concatenate([oracle.tile_rows(n_tokens, t) for t in tiles])


def oracle_rows(case, tiles, rows=None, slack=False):
    """Both oracle modes on the rows of `tiles` (or only `rows` of them):
    (rows, mirror, exact[, slack]).  Many tiles of a named workload are
    evaluated by tests/oracle_worker.py in a CPU-only child process that
    spreads them over the host's cores."""
    import os
    import subprocess
    import sys
    import tempfile
    if rows is None:
        rows = rows_of_tiles(case.n_tokens, tiles)
    rows = np.asarray(rows)
    named = case.name in workloads.CONFIGS and case.seed == workloads.CONFIGS[case.name]["seed"]
    if named and len(tiles) > 4 and not slack:
        here = os.path.dirname(os.path.abspath(__file__))
        with tempfile.TemporaryDirectory() as tmp:
            out = os.path.join(tmp, "oracle.npz")
            env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
            subprocess.run([sys.executable, os.path.join(here, "oracle_worker.py"), case.name, out,
                            *[str(t) for t in tiles]], check=True, env=env)
            z = np.load(out)
            pos = {int(r): i for i, r in enumerate(z["rows"])}
            sel = [pos[int(r)] for r in rows]
            return rows, z["mirror"][sel], z["exact"][sel]
    if slack:
        b, sl = oracle.attention_int8_mirror(case, tiles=tiles, tie_slack=True)
    else:
        b, sl = oracle.attention_int8_mirror(case, tiles=tiles), None
    a = oracle.attention_exact(case, tiles=tiles)
    return (rows, b[rows], a[rows]) + ((sl[rows],) if slack else ())


def check_parity(case, out, tiles=None, label="", rows=None, ref=None, frob_bar=TOL_EXACT_FROB):
    """Compare a GPU output (torch, [N][Hq][256]) with both oracle modes on the
    rows of `tiles` (all tiles when None), or only on `rows` of those tiles;
    `ref` takes a precomputed oracle_rows(...) result; frob_bar=None skips
    the comparison with exact attention (for stress inputs where the int8
    method itself departs from it further).  The bar is the plain
    one: max|d| <= 2e-3 * max|O| against the int8 mirror, for fp32 outputs with
    no allowance at all; a bf16 output is also allowed half a bf16 ulp of
    the larger of its value and the mirror's (its own rounding).  Returns the
    measured errors, with the share of elements whose mirror value depends on
    a near-tie P code (a diagnostic of the oracle's tie window, not part of
    the bar)."""
    n_tiles = (case.n_tokens + 15) // 16
    tiles = list(range(n_tiles)) if tiles is None else sorted(set(tiles))
    if ref is None:
        ref = oracle_rows(case, tiles, rows)
    rows, b, a = ref[:3]
    o = out.float().cpu().numpy()[rows].astype(np.float64)
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    mo = np.abs(b).max()
    d = np.abs(o - b)
    allow = TOL_MIRROR * mo
    if out.dtype == torch.bfloat16:
        allow = allow + bf16_half_ulp(np.maximum(np.abs(b), np.abs(o)))
    frob = float(np.linalg.norm(o - a) / np.linalg.norm(a))
    rel_b = float(d.max() / mo)
    assert np.all(d <= allow), (
        f"{label}: max|d| vs mirror {d.max():.3e} (max|O| {mo:.3e}, rel {rel_b:.3e}) "
        f"at {np.unravel_index(d.argmax(), d.shape)}")
    if frob_bar is not None:
        assert frob <= frob_bar, f"{label}: relative Frobenius vs exact {frob:.3e}"
    res = dict(rel_mirror=rel_b, frob_exact=frob)
    if len(ref) > 3:
        sl = ref[3]
        res.update(tie_elements=float((sl > 0).mean()), max_slack_rel=float(sl.max() / mo))
    return res


def poison_unattended_blocks(d):
    """Point every block of a decode batch's sequences that its query row (the
    last position) does not attend at page 0, whose scales are NaN: a stray
    read of such a block then shows as a non-finite output.  The attended set
    comes from the oracle."""
    for b, L in enumerate(np.asarray(d.seq_lens).tolist()):
        need = min((L + 15) // 16, d.page_tables.shape[1])
        if L <= 0 or need == 0:
            continue
        keys = np.arange(min(L, need * 16))
        att = oracle.attended_mask(np.array([L - 1]), keys, d.window_blocks, d.sink_blocks)[0]
        unattended = np.setdiff1d(np.arange(need), np.unique(keys[att] // 16))
        d.page_tables[b, unattended] = 0
    return d

