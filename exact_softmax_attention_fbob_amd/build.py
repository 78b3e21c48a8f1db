"""Build the gfx950 HIP libraries in-tree (next to this file).

    python -m exact_softmax_attention_fbob_amd.build [--verbose] [--product-only]

* ``libfbob.so``: the product library.  One kernel variant per problem class; it
  reads no environment.
* ``libfbob_tuning.so``: the same sources with ``-DFBOB_TUNING=1``, which also
  compiles the measured alternative variants and lets ``FBOB_TUNE_<KERNEL>``
  environment variables select one at each launch (measurement and the variant
  parity tests only).

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
TUNING_LIB = os.path.join(HERE, "libfbob_tuning.so")
SOURCES = ("fbob_api.hip", "fbob_forward.hip", "fbob_pass1.hip", "fbob_pass2.hip",
           "fbob_grad.hip", "fbob_split.hip")
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


def build(verbose: bool = False, extra=(), tuning: bool = False) -> str:
    """Compile every source to an object in parallel, then link libfbob.so (or,
    with ``tuning``, libfbob_tuning.so)."""
    cc = hipcc()
    lib = TUNING_LIB if tuning else LIB
    if tuning:
        extra = (*extra, "-DFBOB_TUNING=1")
    objdir = os.path.join(HERE, "_build_tuning" if tuning else "_build")
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
    tmp = lib + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(link)}\n{r.stdout}")
    os.replace(tmp, lib)
    if verbose:
        sys.stderr.write(f"[fbob build] {lib} in {time.time() - t0:.1f}s\n")
    return lib


def build_all(verbose: bool = False) -> None:
    """Both libraries, one after the other (each compiles its sources in parallel)."""
    build(verbose=verbose)
    build(verbose=verbose, tuning=True)


if __name__ == "__main__":
    if "--product-only" in sys.argv:
        build(verbose="--verbose" in sys.argv)
    else:
        build_all(verbose="--verbose" in sys.argv)
