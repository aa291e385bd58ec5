"""CPU-only helper for the sampled parity tests: evaluates both oracle modes on
many query tiles of a named workload in parallel worker processes.

    python tests/oracle_worker.py <config> <out.npz> <tile> [<tile> ...]

Runs as its own process (started by the tests with subprocess), so that the
worker pool never shares a process with GPU state.  Writes rows [R], mirror
[R][Hq][256] and exact [R][Hq][256] (fp64) for the rows of the listed tiles.
"""
import multiprocessing as mp
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

_CASE = None


def _one(tile):
    rows = oracle.tile_rows(_CASE.n_tokens, tile)
    b = oracle.attention_int8_mirror(_CASE, tiles=[tile])[rows]
    a = oracle.attention_exact(_CASE, tiles=[tile])[rows]
    return rows, b, a


def main():
    global _CASE
    name, out = sys.argv[1], sys.argv[2]
    tiles = [int(t) for t in sys.argv[3:]]
    _CASE = workloads.make_config(name)
    procs = max(1, min(16, len(os.sched_getaffinity(0)), len(tiles)))
    with mp.get_context("fork").Pool(procs) as pool:
        res = pool.map(_one, tiles)
    rows = np.concatenate([r[0] for r in res])
    np.savez(out, rows=rows, mirror=np.concatenate([r[1] for r in res]),
             exact=np.concatenate([r[2] for r in res]))


if __name__ == "__main__":
    main()
