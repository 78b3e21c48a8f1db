"""ctypes loader for ``libfbob.so`` with the prototypes of ``include/fbob.h``.

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS = {0: "FBOB_OK", 1: "FBOB_ERR_INVALID_ARG", 2: "FBOB_ERR_UNSUPPORTED",
          3: "FBOB_ERR_ALIGNMENT", 4: "FBOB_ERR_ALIAS", 5: "FBOB_ERR_HIP",
          6: "FBOB_ERR_SCRATCH"}

# Every symbol declared in include/fbob.h, with its ctypes prototype.
_i64, _f, _i, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p
_SIZES = [_i, _i64, _i64, _i64, _i64, _i64, _f, _i]  # dtype, B, Hq, Hkv, N, d, tau, causal
PROTOTYPES = {
    "fbob_forward": (_i, _SIZES + [_vp] * 4 + [_vp] * 3 + [_vp]),
    "fbob_backward": (_i, _SIZES + [_vp] * 4 + [_vp] * 2 + [_vp] * 4 + [_vp]),
    "fbob_forward_workspace_size": (_i, _SIZES + [ctypes.POINTER(_i64)]),
    "fbob_forward_ws": (_i, _SIZES + [_vp] * 4 + [_vp] * 3 + [_vp, _i64] + [_vp]),
    "fbob_backward_workspace_size": (_i, _SIZES + [ctypes.POINTER(_i64)]),
    "fbob_backward_ws": (_i, _SIZES + [_vp] * 4 + [_vp] * 2 + [_vp] * 4 + [_vp, _i64] + [_vp]),
    "fbob_bob": (_i, _SIZES + [_vp] * 7 + [_vp] * 3 + [_vp] * 6 + [_vp]),
    "fbob_bob_pass1": (_i, _SIZES + [_vp] * 7 + [_vp] * 3 + [_vp] * 4 + [_vp]),
    "fbob_bob_pass2": (_i, _SIZES + [_vp] * 7 + [_vp] * 4 + [_vp] * 2 + [_vp]),
    "fbob_bob_workspace_size": (_i, _SIZES + [ctypes.POINTER(_i64)]),
    "fbob_bob_ws": (_i, _SIZES + [_vp] * 7 + [_vp] * 3 + [_vp] * 6 + [_vp, _i64] + [_vp]),
    "fbob_bob_noalloc": (_i, _SIZES + [_vp] * 7 + [_vp] * 3 + [_vp] * 6 + [_vp]),
    "fbob_bob_ex": (_i, _SIZES + [_i] + [_vp] * 7 + [_vp] * 3 + [_vp] * 6 + [_vp, _i64] + [_vp]),
    "fbob_strerror": (ctypes.c_char_p, [_i]),
    "fbob_hip_error_string": (ctypes.c_char_p, []),
    "fbob_version": (_i, []),
}


class FbobError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = STATUS.get(status, f"status {status}")
        try:
            lib = load_library()
            msg += ": " + lib.fbob_strerror(status).decode()
            if status == 5:  # FBOB_ERR_HIP: name the HIP error behind it
                msg += f" ({lib.fbob_hip_error_string().decode()})"
        except Exception:  # pragma: no cover - message only
            pass
        super().__init__(msg)


def tuning_library_path() -> str:
    """The measurement build (variants selectable by FBOB_TUNE_* variables)."""
    return os.path.join(_HERE, "libfbob_tuning.so")


@contextlib.contextmanager
def using_library(path: str):
    """Route the binding's calls through another build of the same C ABI (e.g. the
    measurement build) inside the ``with`` block."""
    global _LIB
    prev = _LIB
    _LIB = load_library(path)
    try:
        yield _LIB
    finally:
        _LIB = prev


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle of libfbob.so."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or os.path.join(_HERE, "libfbob.so")
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build the HIP library first "
            "(python -m exact_softmax_attention_fbob_amd.build)")
    # torch first: its HIP runtime (libamdhip64.so.7, which torch loads by another file
    # name) must be in the process before the library asks for libamdhip64.so.7, so that
    # the dynamic loader hands the library that same runtime.  Loaded the other way round,
    # the process would hold two HIP runtimes and the library's would find no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    for name, (res, argt) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = argt
    if path is None:
        _LIB = lib
    return lib
