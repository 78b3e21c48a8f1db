"""Small drivers for hardware-counter runs (run under rocprofv3 on one MI355X).

    python -m exact_softmax_attention_fbob_amd.profiling forward [--workload W] [--launches K]
    python -m exact_softmax_attention_fbob_amd.profiling pass1 [--workload W] [--launches K]
    python -m exact_softmax_attention_fbob_amd.profiling pass2 [--workload W] [--launches K]
    python -m exact_softmax_attention_fbob_amd.profiling copy [--mib M] [--launches K]
    python -m exact_softmax_attention_fbob_amd.profiling record --kernel pass1_kernel \
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv --copy-mib M \
        [--workload W] [--out profiles/pass1_hbm_traffic.json]

`forward`/`pass1`/`pass2` run the forward once and then the chosen kernel K times
on the seeded inputs of a workload (Pass 1 runs once in every case); `copy` runs a plain device-to-device copy of M MiB
(read M MiB, write M MiB) as the calibration kernel for the byte counters;
`record` turns rocprofv3 counter_collection CSVs (FETCH_SIZE / WRITE_SIZE, KiB
per dispatch) into bytes per launch of the chosen kernel, scaled by what the
same counters read for the copy kernel, and writes the JSON that bench.py
reports as roofline.traffic (tagged with a digest of the kernel's sources).
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

KERNEL_SOURCES = {"pass1_kernel": ("fbob_device.hpp", "fbob_pass1.hip"),
                  "pass2_kernel": ("fbob_device.hpp", "fbob_pass2.hip")}


def _code_only(text: str) -> str:
    """C++ source without /* */ and // comments, blank lines or trailing spaces."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_digest(kernel: str) -> str:
    """Digest of the kernel's sources with comments, blank lines and trailing spaces
    removed: a counter record stays valid across comment edits, and only across them."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_softmax_attention_fbob_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _setup(workload):
    import torch
    import workloads
    import exact_softmax_attention_fbob_amd as fb
    w = workloads.WORKLOADS[workload]
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T = {k: torch.from_numpy(v).cuda().to(td) for k, v in workloads.make_inputs(w).items()}
    O, L, D = fb.forward(T["Q"], T["K"], T["V"], T["dO"], w.tau, w.causal)
    args = (T["Q"], T["K"], T["V"], T["dO"], T["UQ"], T["UK"], T["UV"])
    return w, fb, args, O, L, D


def run_pass(which, workload, launches):
    import torch
    w, fb, args, O, L, D = _setup(workload)
    for _ in range(launches if which == "forward" else 0):
        fb.forward(*args[:4], w.tau, w.causal)
    p1 = fb.bob_pass1(*args, O, L, D, w.tau, w.causal)
    for _ in range(launches if which == "pass1" else 0):
        fb.bob_pass1(*args, O, L, D, w.tau, w.causal)
    for _ in range(launches if which == "pass2" else 0):
        fb.bob_pass2(*args, L, D, p1["alpha"], p1["E"], w.tau, w.causal)
    torch.cuda.synchronize()
    print(f"[profiling] {which} x{launches} on {workload} done", flush=True)


def run_copy(mib, launches):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[profiling] copy {mib} MiB x{launches} done", flush=True)


def _per_dispatch(path, counter, name_part):
    """Mean counter value (as reported, KiB) over dispatches whose kernel name
    contains name_part, from a rocprofv3 counter_collection.csv."""
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if name_part not in row.get("Kernel_Name", ""):
                continue
            if row.get("Counter_Name") != counter:
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for '{name_part}' in {path}")
    return sum(vals.values()) / len(vals), len(vals)


def record(a):
    fetch, nf = _per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write, nw = _per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cfetch, _ = _per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cwrite, _ = _per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    known = a.copy_mib * (1 << 20)
    f_scale = known / (cfetch * 1024.0)
    w_scale = known / (cwrite * 1024.0)
    rec = {
        "kernel": a.kernel,
        "workload": a.workload,
        "kernel_source_digest": source_digest(a.kernel),
        "fetch_kib_per_dispatch": fetch,
        "write_kib_per_dispatch": write,
        "dispatches": [nf, nw],
        "copy_calibration": {"mib": a.copy_mib, "fetch_kib": cfetch, "write_kib": cwrite,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "bytes_per_launch": fetch * 1024.0 * f_scale + write * 1024.0 * w_scale,
        "read_bytes_per_launch": fetch * 1024.0 * f_scale,
        "write_bytes_per_launch": write * 1024.0 * w_scale,
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    for name in ("forward", "pass1", "pass2"):
        p = sub.add_parser(name)
        p.add_argument("--workload", default="h12_n16384_d64_bf16_u01")
        p.add_argument("--launches", type=int, default=3)
    p = sub.add_parser("copy")
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--launches", type=int, default=3)
    p = sub.add_parser("record")
    p.add_argument("--kernel", default="pass1_kernel")
    p.add_argument("--copy-kernel", default="copyBuffer")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-fetch", required=True)
    p.add_argument("--copy-write", required=True)
    p.add_argument("--copy-mib", type=int, default=1024)
    p.add_argument("--workload", default="h12_n16384_d64_bf16_u01")
    p.add_argument("--out", default=os.path.join(ROOT, "profiles", "pass1_hbm_traffic.json"))
    a = ap.parse_args()
    if a.cmd in ("forward", "pass1", "pass2"):
        run_pass(a.cmd, a.workload, a.launches)
    elif a.cmd == "copy":
        run_copy(a.mib, a.launches)
    else:
        record(a)


if __name__ == "__main__":
    main()
