"""Benchmark: int8 TOPS of windowed int8 paged prefill attention (hd256) at 32k.

One step = the whole path on one batch of synthetic input already resident in
HBM: Q row quantization, the attention kernel, and the attended-key counts.
Throughput counts 4 * sum_t |A(t)| * 256 * n_q_heads int8 ops per step (the
QK^T and PV multiply-adds of every attended (row, key) pair).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 32k]
                    [--no-cpu-baseline] [--cpu-seconds S] [--copy-calibration]

Prints one JSON line.  Runs on one GPU only.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 TOPS & % of MI355X int8 MFMA peak, hd256 windowed prefill attn at 32k"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix peak, 5.0 POP/s
HBM_PEAK_GBS = 8000.0
ATTN_KERNEL_SOURCES = ["windowed_int8_paged_amd/csrc/wpa_attn.hip", "windowed_int8_paged_amd/csrc/wpa_common.h",
                       "windowed_int8_paged_amd/csrc/wpa_lanes.h"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "prefill_attn_32k_counters.json")


def kernel_source_hash() -> str:
    """Hash of the attention kernels' code with comments and blank space removed, and of
    the compiler flags they are built with, so the recorded traffic counters stay attached
    to a build until its code changes."""
    from windowed_int8_paged_amd import build as wpa_build
    h = hashlib.sha256()
    for p in ATTN_KERNEL_SOURCES:
        text = open(os.path.join(ROOT, p)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    h.update(" ".join(wpa_build.HIP_FLAGS + wpa_build.SOURCE_FLAGS.get("wpa_attn.hip", [])).encode())
    return h.hexdigest()[:16]


def workload_desc(case) -> str:
    win = (f"window {case.window_blocks} blocks + {case.sink_blocks} sink block(s)"
           if case.window_blocks > 0 else "full causal")
    return (f"hd256 prefill attention, N={case.n_tokens}, {case.n_q_heads} q heads / "
            f"{case.n_kv_heads} kv heads, {win}, int8 paged pool of {case.n_pool_pages} "
            f"shuffled 16-token pages, bf16 Q and output")


def copy_calibration(steps: int) -> None:
    """A plain device copy of known size, for scaling rocprofv3 FETCH/WRITE_SIZE."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_direction": n, "launches": steps}), flush=True)


def warm_up(step, args) -> None:
    """The W counted warmup steps, then further untimed steps, queued back to
    back, until args.settle_ms of wall time has passed.  The GPU's clocks rise
    only under continuous load: after an idle gap the first ten or so steps
    of the 32k attention run up to 20% slower (measured per step with HIP
    events), and steps separated by host synchronizations do not settle them."""
    import torch
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def blas_threads() -> int:
    """Threads the oracle's numpy BLAS calls run on."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(case, seconds: float):
    """Time the oracle (as it stands) on a bounded sample of whole query tiles:
    the int8 mirror (mode b) for about two thirds of `seconds`, then exact
    attention (mode a) on the same tiles for the rest."""
    import numpy as np
    import oracle
    threads = blas_threads()
    n_tiles = (case.n_tokens + 15) // 16
    # tiles past the window's fill-up (full-length key lists), else the later half,
    # visited with a stride of 7 so the sample spreads over the sequence
    first = min(n_tiles - 1, max(0, case.window_blocks + 1)) if case.window_blocks > 0 else n_tiles // 2
    span = n_tiles - first
    order = [first + (7 * i) % span for i in range(span)] if span % 7 else list(range(first, n_tiles))

    def ops_of(tiles):
        rows = np.concatenate([oracle.tile_rows(case.n_tokens, t) for t in tiles])
        counts = oracle.mask_counts(case.n_tokens, case.window_blocks, case.sink_blocks)[rows]
        return rows, counts, 4.0 * counts.sum() * 256 * case.n_q_heads

    tiles, t0 = [], time.perf_counter()
    for tile in order:
        oracle.attention_int8_mirror(case, tiles=[tile])
        tiles.append(tile)
        if time.perf_counter() - t0 >= seconds * 2 / 3:
            break
    dt_b = time.perf_counter() - t0
    rows, counts, ops_b = ops_of(tiles)
    tiles_a, t0 = [], time.perf_counter()
    for tile in tiles:
        oracle.attention_exact(case, tiles=[tile])
        tiles_a.append(tile)
        if time.perf_counter() - t0 >= seconds / 3:
            break
    dt_a = time.perf_counter() - t0
    _, _, ops_a = ops_of(tiles_a)
    return {
        "value": ops_b / dt_b / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
        "sample": f"int8-mirror oracle (mode b, numpy fp64) on {len(tiles)} of {n_tiles} query tiles "
                  f"({len(rows)} rows x {case.n_q_heads} heads, {int(counts.sum())} attended keys/head) "
                  f"of the same workload, {dt_b:.1f} s; host cpu_count {os.cpu_count()}",
        "exact_value": ops_a / dt_a / 1e12,
        "exact_sample": f"exact-attention oracle (mode a, numpy fp64) on {len(tiles_a)} of the same tiles, "
                        f"{dt_a:.1f} s, same op count per tile",
    }


def bench_kv_write(args):
    """The KV-pool writer on the 32k workload's shape: 32768 tokens x 4 KV heads of
    bf16 K and V quantized into a 2048-page pool.  HBM-bound: the roofline is the
    bytes it must move (bf16 rows in, int8 rows and float scales out, the slots)."""
    import numpy as np
    import torch
    import windowed_int8_paged_amd as wpa
    import workloads

    n, hkv, pages = 32768, 4, 2048
    kb, vb, _, _, slots, kp, vp, ks, vs = workloads.make_kv_rows(n, hkv, pages, seed=1003)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k, v, sl = bf(kb), bf(vb), dev(slots)
    kp, vp, ks, vs = dev(kp), dev(vp), dev(ks), dev(vs)
    call = lambda: wpa.kv_write_i8(k, v, sl, kp, vp, ks, vs)
    warm_up(call, args)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    nbytes = 2 * n * hkv * 256 * 2 + 4 * n + 2 * n * hkv * (256 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "KV-pool write GB/s (bf16 K/V rows -> int8 pool pages + per-token scales)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16->int8", "data": "synthetic",
        "config": {"workload": f"KV-pool write, {n} tokens x {hkv} KV heads x 256 bf16 K and V into a "
                               f"{pages}-page pool at shuffled slots", "bytes_per_call": nbytes},
        "kernel_ms": {"kv_write_i8": round(ms, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "kv_write_i8"},
    }
    if not args.no_cpu_baseline:
        import oracle
        m = 4096  # the oracle's writer on the first 4096 tokens of the same inputs
        _, _, kf, vf, _, kp0, vp0, ks0, vs0 = workloads.make_kv_rows(n, hkv, pages, seed=1003)
        t0 = time.perf_counter()
        oracle.kv_write_i8(kf[:m], vf[:m], slots[:m], kp0, vp0, ks0, vs0)
        dt = time.perf_counter() - t0
        mbytes = 2 * m * hkv * 256 * 2 + 4 * m + 2 * m * hkv * (256 + 4)
        res["cpu_baseline"] = {"value": round(mbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"oracle writer (numpy) on the first {m} of {n} tokens, {dt:.2f} s, "
                                         f"bytes counted as for the GPU call (the oracle also copies the pool)"}
    print(json.dumps(res), flush=True)


def bench_chunk(args):
    """Chunked prefill past the pages' 64k batched limit: the query rows
    65536 .. 69631 (16 q heads / 4 KV heads, window 256 blocks + 1 sink block)
    over a cache of 69632 tokens already in the pool; quantize + attention."""
    import numpy as np
    import torch
    import windowed_int8_paged_amd as wpa
    import workloads

    q_start, n = 65536, 4096
    case = workloads.make_case(name="chunk", n_tokens=q_start + n, n_q_heads=16, n_kv_heads=4, window_blocks=256,
                               sink_blocks=1, seed=1006)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = torch.from_numpy(case.q_bf16[q_start:].view(np.int16)).cuda().view(torch.bfloat16)
    kp, vp, ks, vs, pt = (dev(a) for a in (case.k_pool, case.v_pool, case.k_scale, case.v_scale, case.page_table))
    q_i8 = torch.empty((n, 16, 256), dtype=torch.int8, device="cuda")
    q_scale = torch.empty((n, 16), dtype=torch.float32, device="cuda")
    out = torch.empty((n, 16, 256), dtype=torch.bfloat16, device="cuda")
    counts = wpa.mask_counts_chunk(q_start, n, 256, 1)
    torch.cuda.synchronize()
    keys = int(counts.to(torch.int64).sum().item())
    ops = 4.0 * keys * 256 * 16

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        wpa.quantize_q_rows(q, q_i8, q_scale)
        if ev is not None:
            ev[1].record()
        wpa.prefill_attn_i8_chunk(q_start, q_i8, q_scale, kp, vp, ks, vs, pt, 256, 1, case.softmax_scale, out=out)
        if ev is not None:
            ev[2].record()

    warm_up(step, args)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms = wall * 1e3 / args.steps
    res = {
        "metric": "int8 TOPS, hd256 windowed prefill attn, 4096-row chunk at position 65536",
        "value": round(ops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "chunked prefill: query rows 65536..69631 of a 69632-token sequence, 16 q heads / "
                               "4 kv heads, window 256 blocks + 1 sink block, int8 paged pool of 4352 shuffled "
                               "16-token pages, bf16 Q and output", "attended_keys": keys, "int8_ops_per_step": ops},
        "kernel_ms": {"quantize_q_rows": round(quant_ms, 4), "prefill_attn_i8_chunk": round(attn_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(ops / (attn_ms * 1e-3) / 1e12, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TOPS", "frac": round(ops / (attn_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                     "traffic": None, "kernel": "prefill_attn_i8_chunk"},
    }
    if not args.no_cpu_baseline:
        import oracle
        tiles, t1 = [], time.perf_counter()
        for tile in range(q_start // 16, (q_start + n) // 16, 37):
            oracle.attention_int8_mirror(case, tiles=[tile])
            tiles.append(tile)
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t1
        rows = np.concatenate([oracle.tile_rows(case.n_tokens, t) for t in tiles])
        cops = 4.0 * oracle.mask_counts(case.n_tokens, 256, 1)[rows].sum() * 256 * 16
        res["cpu_baseline"] = {"value": cops / dt / 1e12, "unit": "TOPS", "cores": blas_threads(), "kind": "oracle",
                               "sample": f"int8-mirror oracle on {len(tiles)} of {n // 16} chunk tiles, {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def bench_decode(args):
    """Split-KV decode: one new token for each of 64 sequences at position 32767
    (16 q heads / 4 kv heads, window 256 blocks + 1 sink block), every block of
    every sequence on a page of its own (4.3 GB of pool, of which each step
    reads the 257 pages per sequence its token attends).  HBM-bound: the roofline is the K
    and V rows plus scales of every attended key (plus Q and out)."""
    import numpy as np
    import torch
    import windowed_int8_paged_amd as wpa
    import workloads

    B, L, hq, hkv, W, S = 64, 32768, 16, 4, 256, 1
    d = workloads.make_decode_batch([L] * B, hq, hkv, W, S, seed=1007, owned_pages=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = torch.from_numpy(d.q_bf16.view(np.int16)).cuda().view(torch.bfloat16)
    kp, vp, ks, vs = dev(d.k_pool), dev(d.v_pool), dev(d.k_scale), dev(d.v_scale)
    tables, lens = dev(d.page_tables), dev(d.seq_lens)
    q_i8 = torch.empty((B, hq, 256), dtype=torch.int8, device="cuda")
    q_scale = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, hq, 256), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((wpa.decode_workspace_bytes(B, hq, tables.shape[1], W, S),), dtype=torch.uint8, device="cuda")
    keys = int(wpa.mask_counts_chunk(L - 1, 1, W, S).item())  # keys the last position attends

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        wpa.quantize_q_rows(q, q_i8, q_scale)
        if ev is not None:
            ev[1].record()
        wpa.decode_attn_i8(q_i8, q_scale, kp, vp, ks, vs, tables, lens, W, S, d.softmax_scale, out=out,
                           workspace=ws)
        if ev is not None:
            ev[2].record()

    warm_up(step, args)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    nbytes = B * keys * hkv * (2 * 256 + 2 * 4) + B * hq * (256 + 4) + B * hq * 256 * 2
    gbs = nbytes / (dec_ms * 1e-3) / 1e9
    res = {
        "metric": "decode GB/s (int8 split-KV decode over the paged pool, one token for each of 64 sequences)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"decode, {B} sequences at position {L - 1}, {hq} q heads / {hkv} kv heads, window "
                               f"{W} blocks + {S} sink block, every block on its own page, {keys // 16} pages read per sequence",
                   "attended_keys_per_sequence": keys, "bytes_per_step": nbytes,
                   "tokens_per_s": round(B / (wall / args.steps), 1)},
        "kernel_ms": {"quantize_q_rows": round(quant_ms, 4), "decode_attn_i8": round(dec_ms, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "decode_attn_i8"},
    }
    if not args.no_cpu_baseline:
        import oracle
        t1, done = time.perf_counter(), 0
        for b in range(B):
            case = workloads.decode_row_case(d, b)
            oracle.attention_int8_mirror(case, tiles=[(L - 1) // 16])
            done += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t1
        cb = done * keys * hkv * (2 * 256 + 2 * 4)
        res["cpu_baseline"] = {"value": round(cb / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
                               "kind": "oracle", "sample": f"int8-mirror oracle, {done} of {B} sequences (a whole "
                                                           f"16-row tile each), {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="after the warmup steps, further untimed steps for this long (clock settling)")
    ap.add_argument("--config", default="32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--q-path", choices=["fused", "separate"], default="fused",
                    help="attention: fused = wpa_prefill_attn_fused_q (Q quantized inside the attention kernels); "
                         "separate = wpa_quantize_q_rows then wpa_prefill_attn_i8.  The other path is timed "
                         "after the main steps and reported beside them")
    ap.add_argument("--op", choices=["attention", "kv_write", "chunk", "decode"], default="attention",
                    help="attention: the headline step; kv_write: the KV-pool writer at the 32k shape; "
                         "chunk: a 4096-row prefill chunk at position 65536 over a 69632-token cache; "
                         "decode: one token for each of 64 sequences at position 32767")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(sharding by KV head or by query range is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(max(1, args.steps))
        return
    if args.op == "kv_write":
        bench_kv_write(args)
        return
    if args.op == "chunk":
        bench_chunk(args)
        return
    if args.op == "decode":
        bench_decode(args)
        return

    import windowed_int8_paged_amd as wpa
    import workloads

    case = workloads.make_config(args.config)
    N, Hq = case.n_tokens, case.n_q_heads
    print(f"[bench] config {args.config}: {workload_desc(case)}", file=sys.stderr, flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = torch.from_numpy(case.q_bf16.view(np.int16)).cuda().view(torch.bfloat16)
    k_pool, v_pool = dev(case.k_pool), dev(case.v_pool)
    k_scale, v_scale, page_table = dev(case.k_scale), dev(case.v_scale), dev(case.page_table)
    q_i8 = torch.empty((N, Hq, 256), dtype=torch.int8, device="cuda")
    q_scale = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((N, Hq, 256), dtype=torch.bfloat16, device="cuda")
    counts = torch.empty((N,), dtype=torch.int32, device="cuda")

    def attn(ev=None):
        wpa.prefill_attn_i8(q_i8, q_scale, k_pool, v_pool, k_scale, v_scale, page_table,
                            case.window_blocks, case.sink_blocks, case.softmax_scale, out=out)

    def step_separate(ev=None):
        if ev is not None:
            ev[0].record()
        wpa.quantize_q_rows(q, q_i8, q_scale)
        if ev is not None:
            ev[1].record()
        attn()
        if ev is not None:
            ev[2].record()
        wpa.mask_counts(N, case.window_blocks, case.sink_blocks, counts=counts)
        if ev is not None:
            ev[3].record()

    def step_fused(ev=None):
        if ev is not None:
            ev[0].record()
            ev[1].record()
        wpa.prefill_attn_fused_q(q, k_pool, v_pool, k_scale, v_scale, page_table, case.window_blocks,
                                 case.sink_blocks, case.softmax_scale, out=out)
        if ev is not None:
            ev[2].record()
        wpa.mask_counts(N, case.window_blocks, case.sink_blocks, counts=counts)
        if ev is not None:
            ev[3].record()

    def attn_only(ev=None):
        if ev is not None:
            ev[0].record()
            ev[1].record()
        attn()
        if ev is not None:
            ev[2].record()
            ev[3].record()

    def timed(step, n):
        """Wall-clock ms per step over n steps, and the mean HIP-event spans
        (quantize, attention, mask counts) of a step."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        spans = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(3)]
        per_step = [e[0].elapsed_time(e[3]) for e in evs]
        print(f"[bench] {step.__name__}: step ms " + " ".join(f"{x:.3f}" for x in per_step),
              file=sys.stderr, flush=True)
        return wall * 1e3 / n, spans

    main_step, other_step = ((step_fused, step_separate) if args.q_path == "fused"
                             else (step_separate, step_fused))
    other_step()
    torch.cuda.synchronize()
    # before the warm-up: the first torch reduction loads its kernels, a pause
    # long enough for the clocks to drop again
    total_keys = int(counts.to(torch.int64).sum().item())
    ops = 4.0 * total_keys * 256 * Hq
    warm_up(main_step, args)

    # the timed steps of the chosen user path; then, untimed for `value`, the
    # int8-Q attention launch alone and the other path
    ms_per_step, (quant_ms, main_attn_ms, mask_ms) = timed(main_step, args.steps)
    attn_ms = timed(attn_only, args.steps)[1][1]
    other_ms, (other_quant_ms, other_attn_ms, _) = timed(other_step, args.steps)
    value = ops / (ms_per_step * 1e-3) / 1e12
    if args.q_path == "fused":
        fused_ms, sep_quant_ms = main_attn_ms, other_quant_ms
    else:
        fused_ms, sep_quant_ms = other_attn_ms, quant_ms
    # the roofline kernel is the attention launch of the timed path, timed by
    # HIP events on the stream it runs on
    roof_ms = main_attn_ms
    roof_kernel = "prefill_attn_fused_q" if args.q_path == "fused" else "prefill_attn_i8"
    roof_tops = ops / (roof_ms * 1e-3) / 1e12

    # HBM traffic and the clock under this load come from rocprofv3 counters
    # of the same kernel code (FETCH_SIZE/WRITE_SIZE scaled by a plain copy;
    # GRBM_GUI_ACTIVE over the dispatch's duration), recorded with the hash of
    # the source they were taken on: a changed kernel reports null
    traffic = clock_mhz = None
    if os.path.exists(COUNTERS_FILE):
        t = json.load(open(COUNTERS_FILE))
        if (t.get("kernel_source_hash") == kernel_source_hash() and t.get("config") == args.config
                and t.get("kernel") == roof_kernel):
            traffic = t.get("hbm_bytes_per_launch")
            clock_mhz = t.get("clock_mhz")

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": workload_desc(case), "name": args.config, "n_tokens": N,
                   "n_q_heads": Hq, "n_kv_heads": case.n_kv_heads, "head_dim": 256,
                   "window_blocks": case.window_blocks, "sink_blocks": case.sink_blocks,
                   "attended_keys": total_keys, "int8_ops_per_step": ops, "parallelism": "single-gpu"},
        "pct_of_int8_peak_step": round(100 * value / PEAK_INT8_TOPS, 2),
        "q_path": args.q_path,
        "kernel_ms": {"prefill_attn_fused_q": round(fused_ms, 4), "quantize_q_rows": round(sep_quant_ms, 4),
                      "prefill_attn_i8": round(attn_ms, 4), "mask_counts": round(mask_ms, 4)},
        "other_q_path_ms_per_step": round(other_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(roof_tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TOPS", "frac": round(roof_tops / PEAK_INT8_TOPS, 4),
                     "traffic": traffic, "kernel": roof_kernel, "kernel_ms": round(roof_ms, 4),
                     "clock_mhz": round(clock_mhz, 1) if clock_mhz else None, "clock_source": "rocprofv3 counters",
                     "frac_at_clock": round(roof_tops / (PEAK_INT8_TOPS * clock_mhz / 2400.0), 4) if clock_mhz else None,
                     "kernel_source_hash": kernel_source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
