"""Write the oracle's dK~ and dV~ at seeded key columns of the two largest workloads.

    python tests/golden/make_large_columns.py [--workers 8] [--only WORKLOAD]

A column of dK~ or dV~ sums over every query row, and each row enters through its
four scalars (L, D, alpha, E), which need that row's products with every key: an
O(N^2 d) pass per head that takes minutes of host time at these sizes, too long to
repeat in a GPU test.  This script runs that pass once with the fp64 oracle
(``oracle.row_scalars`` over all rows, row blocks spread over worker processes),
then evaluates the selected columns exactly (``oracle.bob_columns_at``), and stores
them under ``tests/golden/large_columns_<workload>.npz``.  It calls only ``oracle``
and ``workloads``; no value comes from the GPU.

Stored per workload: the checked heads, the column indices (seeded draw plus the
first and last key), dK~ and dV~ at those columns rounded to float32 (a relative
change below 6e-8, far under the 2e-2 comparison bar), and a SHA-256 digest of the
seeded inputs of those heads so that a test can confirm it regenerated the same
inputs.
"""

from __future__ import annotations

import os

# One BLAS thread per worker process (set before numpy is imported).
for _v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

import argparse  # noqa: E402
import json  # noqa: E402
import multiprocessing as mp  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

# workload -> (heads checked, columns per head, row block of the scalar pass)
PLAN = {
    "h8_n65536_d128_bf16_qk2": (list(range(8)), 64, 128),
    "h1_n262144_d64_bf16": ([0], 256, 64),
}
COLUMN_SEED = 4242

_HEAD = {}  # the current head's float64 inputs, inherited by forked workers


def out_path(name: str) -> str:
    return os.path.join(HERE, f"large_columns_{name}.npz")


def pick_columns(N: int, n_cols: int, flat_head: int) -> np.ndarray:
    rng = np.random.default_rng([COLUMN_SEED, N, flat_head])
    cols = rng.choice(np.arange(1, N - 1), size=n_cols - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], cols])).astype(np.int64)


def _scalars_of_block(job):
    r0, r1, tau, causal = job
    a = _HEAD["args"]
    return r0, oracle.row_scalars(*a, tau, np.arange(r0, r1), causal)


def run(name: str, workers: int) -> None:
    w = workloads.WORKLOADS[name]
    heads, n_cols, rb = PLAN[name]
    t0 = time.time()
    inp = workloads.make_inputs(w)
    digest = workloads.input_digest(inp, heads)
    print(f"[golden] {name}: inputs drawn ({time.time() - t0:.1f} s), digest {digest[:16]}",
          flush=True)
    cols_all, dk_all, dv_all = [], [], []
    for f in heads:
        b, h = divmod(f, w.H)
        _HEAD["args"] = [inp[k][b, h].astype(np.float64) for k in workloads.TENSORS]
        jobs = [(r0, min(w.N, r0 + rb), w.tau, w.causal) for r0 in range(0, w.N, rb)]
        rs = {k: np.empty(w.N) for k in ("L", "D", "alpha", "E")}
        th = time.time()
        with mp.get_context("fork").Pool(workers) as pool:
            for k_done, (r0, part) in enumerate(pool.imap_unordered(_scalars_of_block, jobs, 4)):
                for k in rs:
                    rs[k][r0:r0 + len(part[k])] = part[k]
                if (k_done + 1) % max(1, len(jobs) // 8) == 0:
                    print(f"[golden] {name} head {f}: {k_done + 1}/{len(jobs)} row blocks "
                          f"({time.time() - th:.0f} s)", flush=True)
        cols = pick_columns(w.N, n_cols, f)
        c = oracle.bob_columns_at(*_HEAD["args"], w.tau, cols, rs["L"], rs["D"], rs["alpha"],
                                  rs["E"], w.causal)
        cols_all.append(cols)
        dk_all.append(c["dKt"].astype(np.float32))
        dv_all.append(c["dVt"].astype(np.float32))
        print(f"[golden] {name} head {f}: done in {time.time() - th:.0f} s, "
              f"max|dK~| {np.abs(c['dKt']).max():.3e} max|dV~| {np.abs(c['dVt']).max():.3e}",
              flush=True)
    meta = {"workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype,
            "seed": w.seed, "scale_u": w.scale_u, "scale_qk": w.scale_qk, "causal": w.causal,
            "tau": w.tau, "column_seed": COLUMN_SEED,
            "oracle": "row_scalars over all rows, then bob_columns_at (fp64 numpy)"}
    np.savez(out_path(name), heads=np.array(heads, np.int64), cols=np.stack(cols_all),
             dKt=np.stack(dk_all), dVt=np.stack(dv_all), input_sha256=np.array(digest),
             meta=np.array(json.dumps(meta)))
    print(f"[golden] wrote {out_path(name)} ({time.time() - t0:.0f} s)", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--only", default=None)
    a = ap.parse_args()
    for name in PLAN:
        if a.only is None or a.only == name:
            run(name, a.workers)


if __name__ == "__main__":
    main()
