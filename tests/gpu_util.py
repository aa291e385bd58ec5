"""Helpers for the GPU parity tests: upload a seeded case, run the library
through its C ABI, and compare with the oracle at the stated tolerances."""
import numpy as np
import torch

import oracle

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


def check_parity(case, out, tiles=None, label="", rows=None):
    """Compare a GPU output (torch, [N][Hq][256]) with both oracle modes on the
    rows of `tiles` (all tiles when None), or only on `rows` of those tiles.
    Returns the measured errors."""
    n_tiles = (case.n_tokens + 15) // 16
    tiles = list(range(n_tiles)) if tiles is None else sorted(set(tiles))
    if rows is None:
        rows = rows_of_tiles(case.n_tokens, tiles)
    rows = np.asarray(rows)
    o = out.float().cpu().numpy()[rows].astype(np.float64)
    b, slack = oracle.attention_int8_mirror(case, tiles=tiles, tie_slack=True)
    b, slack = b[rows], slack[rows]
    a = oracle.attention_exact(case, tiles=tiles)[rows]
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    mo = np.abs(b).max()
    d = np.abs(o - b)
    # codes whose float32 argument sits within rounding error of a .5 tie may
    # round either way; their whole effect is allowed on top of the bar
    allow = TOL_MIRROR * mo + slack
    if out.dtype == torch.bfloat16:
        allow = allow + bf16_half_ulp(b)
    worst = float((d - allow).max())
    frob = float(np.linalg.norm(o - a) / np.linalg.norm(a))
    rel_b = float(d.max() / mo)
    assert np.all(d <= allow), (
        f"{label}: max|d| vs mirror {d.max():.3e} (max|O| {mo:.3e}, rel {rel_b:.3e}) "
        f"at {np.unravel_index(d.argmax(), d.shape)}")
    assert frob <= TOL_EXACT_FROB, f"{label}: relative Frobenius vs exact {frob:.3e}"
    return dict(rel_mirror=rel_b, frob_exact=frob, worst_margin=worst,
                max_slack_rel=float(slack.max() / mo))
