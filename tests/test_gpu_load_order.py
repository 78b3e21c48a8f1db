"""The binding loads the library only after torch, so the process holds one HIP runtime
(torch's bundled copy, which the library's libamdhip64.so.7 request then resolves to).
This runs a fresh interpreter that loads the library before it touches torch itself
(as a test fixture that switches libraries does), then computes on the GPU."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = r"""
import sys
sys.path.insert(0, sys.argv[1])
import exact_softmax_attention_fbob_amd as fb
from exact_softmax_attention_fbob_amd import _lib
for path in (_lib.tuning_library_path(), None):
    lib = _lib.load_library(path)          # before this script imports torch
    import torch
    x = torch.randn(1, 2, 130, 64, device="cuda").to(torch.bfloat16)
    with _lib.using_library(path or fb.library_path()):
        O, L, _ = fb.forward(x, x, x, None, 0.125, False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all())
    print("ok", path or "product", flush=True)
"""


def test_library_loaded_before_torch_shares_torchs_hip_runtime():
    print("[load-order] fresh interpreter", flush=True)
    r = subprocess.run([sys.executable, "-c", CODE, ROOT], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok") == 2, r.stdout
