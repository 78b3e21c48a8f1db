"""Build the gfx950 HIP library ``libfbob.so`` in-tree (next to this file).

    python -m exact_softmax_attention_fbob_amd.build [--verbose]

hipcc cross-compiles for gfx950 without a GPU present.  Packed fp32 VALU
instructions are disabled in device code (``-packed-fp32-ops``); hipcc's host
pass warns that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfbob.so")
SOURCES = ("fbob_api.hip", "fbob_forward.hip", "fbob_pass1.hip", "fbob_pass2.hip",
           "fbob_grad.hip")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags(extra=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", *extra]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel, then link libfbob.so."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"[fbob build] {src} failed:\n{' '.join(cmd)}\n{out}\n")
        elif verbose and out.strip():
            sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError(f"HIP build failed for {failed}")
    tmp = LIB + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(link)}\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(f"[fbob build] {LIB} in {time.time() - t0:.1f}s\n")
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
