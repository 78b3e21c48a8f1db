"""Exact backward-over-backward (BoB) of softmax attention on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/fbob.h`` (``libfbob.so``, built
in-tree by ``exact_softmax_attention_fbob_amd.build``).  This module only
marshals arguments: it checks shapes, dtypes, devices and contiguity, allocates
the output tensors with torch (device memory) and passes raw pointers and
torch's current HIP stream to the library.  Every step of the computation runs
in the library's HIP kernels; there is no fallback path.

Entry points (same names as the C ABI):
    forward(Q, K, V, dO, tau, causal)              -> O, L, D   (dO=None: O, L, None)
    backward(Q, K, V, dO, O, L, tau, causal)       -> dict(dQ, dK, dV, D)
    backward_ws(..., workspace)                     -> as backward; small problems split
    bob(Q, K, V, dO, UQ, UK, UV, O, L, D, ...)     -> dict(dQt, dKt, dVt, ddOt, alpha, E)
    bob_pass1(...)                                  -> dict(dQt, ddOt, alpha, E)
    bob_pass2(..., alpha, E)                        -> dict(dKt, dVt)
    bob_ws(..., workspace)                          -> as bob; small problems split
    bob_workspace_size(Q, K, tau, causal)           -> bytes bob_ws can use
    bob_ex(..., flags, workspace)                   -> as bob_ws, with FLAG_* options
    bob_noalloc(..., out)                           -> as bob_ws, static scratch
Shapes: Q, dO, U_Q: [B, Hq, N, d]; K, V, U_K, U_V: [B, Hkv, N, d]; L, D, alpha,
E: [B, Hq, N]; all outputs float32.  ``FBOB_SYNC_DEBUG=1`` in the environment (read at
import) makes every call wait for its stream and name itself in a device error.  ``autograd.attention`` wraps forward,
backward and bob as a twice-differentiable torch operation.
"""

from __future__ import annotations

import ctypes
import math
import os

from ._lib import FbobError, load_library, STATUS  # noqa: F401

__all__ = ["forward", "forward_ws", "forward_workspace_size", "backward", "backward_ws",
           "backward_workspace_size", "bob", "bob_pass1", "bob_pass2", "bob_ws", "bob_ex",
           "bob_noalloc", "bob_workspace_size", "FLAG_FP32_ROW_SUMS", "load_library",
           "FbobError", "library_path", "version"]

# fbob_bob_ex option bits (include/fbob.h): bf16 d = 64 row sums alpha, E' in fp32
FLAG_FP32_ROW_SUMS = 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libfbob.so")


def version() -> int:
    return load_library().fbob_version()


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype == torch.float32:
        return 0
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _check_inputs(Q, K, V, dO, UQ=None, UK=None, UV=None):
    ins = [x for x in (Q, K, V, dO, UQ, UK, UV) if x is not None]
    for x in ins:
        if not x.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if x.device != Q.device:
            raise ValueError("all tensors must be on the same GPU")
        if not x.is_contiguous():
            raise ValueError("all tensors must be contiguous ([B, H, N, d], d fastest)")
        if x.dtype != Q.dtype:
            raise TypeError("the seven inputs must share one dtype")
        if x.dim() != 4:
            raise ValueError("inputs are 4-D [B, H, N, d]")
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    for x in (Q, dO, UQ):
        if x is not None and tuple(x.shape) != (B, Hq, N, d):
            raise ValueError(f"expected query-side shape {(B, Hq, N, d)}, got {tuple(x.shape)}")
    for x in (K, V, UK, UV):
        if x is not None and tuple(x.shape) != (B, Hkv, N, d):
            raise ValueError(f"expected key-side shape {(B, Hkv, N, d)}, got {tuple(x.shape)}")
    return B, Hq, Hkv, N, d


def _check_f32(x, shape, name, dev):
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if x.device != dev:
        raise ValueError(f"{name} must be on the inputs' GPU ({dev})")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    """torch's current stream on the inputs' device."""
    return ctypes.c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


# FBOB_SYNC_DEBUG=1 (read once, at import): after every library call the binding waits
# for the call's stream, so that an asynchronous device error is reported by the call
# that launched the faulting kernel (named in the message) instead of by a later one.
# Debugging aid only: it serialises host and device (and is skipped while the stream is
# being captured into a HIP graph).  The C library itself reads no environment.
_SYNC_DEBUG = os.environ.get("FBOB_SYNC_DEBUG", "") not in ("", "0")


def _call(dev, fn, *args):
    """Call a library entry point with the inputs' device current (the kernels launch
    on the current device, into the given stream of that device)."""
    torch = _torch()
    with torch.cuda.device(dev):
        st = fn(*args)
        if st == 0 and _SYNC_DEBUG and not torch.cuda.is_current_stream_capturing():
            try:
                torch.cuda.current_stream(dev).synchronize()
            except RuntimeError as e:
                raise RuntimeError(f"{getattr(fn, '__name__', 'fbob call')}: device error "
                                   f"after launch ({e})") from e
    if st != 0:
        raise FbobError(st)


def _tau(tau, d):
    return ctypes.c_float(1.0 / math.sqrt(d) if tau is None else float(tau))


def forward(Q, K, V, dO=None, tau=None, causal=False):
    """O, L, D for the BoB row state (C ABI ``fbob_forward``).

    With ``dO=None`` only the attention forward runs and D is returned as None.
    """
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO)
    O = torch.empty((B, Hq, N, d), dtype=torch.float32, device=Q.device)
    L = torch.empty((B, Hq, N), dtype=torch.float32, device=Q.device)
    D = None if dO is None else torch.empty((B, Hq, N), dtype=torch.float32, device=Q.device)
    _call(Q.device, lib.fbob_forward, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), None if dO is None else _p(dO), _p(O), _p(L),
          None if D is None else _p(D), _stream(Q.device))
    return O, L, D


def forward_workspace_size(Q, K, tau=None, causal=False) -> int:
    """Bytes of device workspace ``forward_ws`` can use for this problem (C ABI
    ``fbob_forward_workspace_size``); 0 when the problem fills the GPU unsplit."""
    lib = load_library()
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    out = ctypes.c_int64(0)
    st = lib.fbob_forward_workspace_size(_dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
                                         int(bool(causal)), ctypes.byref(out))
    if st != 0:
        raise FbobError(st)
    return int(out.value)


def forward_ws(Q, K, V, dO=None, tau=None, causal=False, workspace=None):
    """``forward`` with a caller-owned workspace (C ABI ``fbob_forward_ws``): problems too
    small to fill the GPU split each row tile's key sweep over more work-groups.
    ``workspace`` is a contiguous GPU tensor of at least ``forward_workspace_size`` bytes;
    None allocates one with torch.  Returns (O, L, D) like ``forward``."""
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO)
    dev = Q.device
    if workspace is None:
        need = forward_workspace_size(Q, K, tau, causal)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' GPU")
    nbytes = workspace.numel() * workspace.element_size()
    O = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    L = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    D = None if dO is None else torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    _call(dev, lib.fbob_forward_ws, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), None if dO is None else _p(dO), _p(O), _p(L),
          None if D is None else _p(D), _p(workspace), nbytes, _stream(dev))
    return O, L, D


def backward(Q, K, V, dO, O, L, tau=None, causal=False):
    """First-order gradients dQ, dK, dV and the row scalar D (C ABI ``fbob_backward``).

    O and L come from ``forward`` on the same (Q, K, V); the returned D completes
    the row state (O, L, D) that ``bob`` takes.  dK and dV have the key/value heads'
    shape (grouped query heads are summed).
    """
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO)
    dev = Q.device
    _check_f32(O, (B, Hq, N, d), "O", dev)
    _check_f32(L, (B, Hq, N), "L", dev)
    out = dict(dQ=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               dK=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               dV=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               D=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    _call(dev, lib.fbob_backward, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), _p(dO), _p(O), _p(L),
          _p(out["dQ"]), _p(out["dK"]), _p(out["dV"]), _p(out["D"]), _stream(dev))
    return out


def backward_workspace_size(Q, K, tau=None, causal=False) -> int:
    """Bytes of device workspace ``backward_ws`` can use for this problem (C ABI
    ``fbob_backward_workspace_size``); 0 when the problem fills the GPU unsplit."""
    lib = load_library()
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    out = ctypes.c_int64(0)
    st = lib.fbob_backward_workspace_size(_dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
                                          int(bool(causal)), ctypes.byref(out))
    if st != 0:
        raise FbobError(st)
    return int(out.value)


def backward_ws(Q, K, V, dO, O, L, tau=None, causal=False, workspace=None):
    """``backward`` with a caller-owned workspace (C ABI ``fbob_backward_ws``): problems
    too small to fill the GPU split their sweeps over more work-groups.  ``workspace`` is a
    contiguous GPU tensor of at least ``backward_workspace_size`` bytes; None allocates
    one with torch.  Returns the same dict as ``backward``."""
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO)
    dev = Q.device
    _check_f32(O, (B, Hq, N, d), "O", dev)
    _check_f32(L, (B, Hq, N), "L", dev)
    if workspace is None:
        need = backward_workspace_size(Q, K, tau, causal)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' GPU")
    nbytes = workspace.numel() * workspace.element_size()
    out = dict(dQ=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               dK=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               dV=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               D=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    _call(dev, lib.fbob_backward_ws, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), _p(dO), _p(O), _p(L),
          _p(out["dQ"]), _p(out["dK"]), _p(out["dV"]), _p(out["D"]), _p(workspace), nbytes,
          _stream(dev))
    return out


def _row_state(O, L, D, B, Hq, N, d, dev):
    _check_f32(O, (B, Hq, N, d), "O", dev)
    _check_f32(L, (B, Hq, N), "L", dev)
    _check_f32(D, (B, Hq, N), "D", dev)


def bob(Q, K, V, dO, UQ, UK, UV, O, L, D, tau=None, causal=False, out=None):
    """Exact BoB outputs (C ABI ``fbob_bob``: Pass 1 then Pass 2 on one stream).

    ``out`` may supply preallocated float32 outputs (dict with the six keys).
    """
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO, UQ, UK, UV)
    dev = Q.device
    _row_state(O, L, D, B, Hq, N, d, dev)
    if out is None:
        out = dict(dQt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
                   dKt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
                   dVt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
                   ddOt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
                   alpha=torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
                   E=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    else:
        for k, shp in (("dQt", (B, Hq, N, d)), ("dKt", (B, Hkv, N, d)), ("dVt", (B, Hkv, N, d)),
                       ("ddOt", (B, Hq, N, d)), ("alpha", (B, Hq, N)), ("E", (B, Hq, N))):
            _check_f32(out[k], shp, k, dev)
    _call(dev, lib.fbob_bob, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d), int(bool(causal)),
          _p(Q), _p(K), _p(V), _p(dO), _p(UQ), _p(UK), _p(UV), _p(O), _p(L), _p(D),
          _p(out["dQt"]), _p(out["dKt"]), _p(out["dVt"]), _p(out["ddOt"]),
          _p(out["alpha"]), _p(out["E"]), _stream(dev))
    return out


def bob_pass1(Q, K, V, dO, UQ, UK, UV, O, L, D, tau=None, causal=False):
    """Pass 1 alone (C ABI ``fbob_bob_pass1``): dQt, ddOt, alpha, E."""
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO, UQ, UK, UV)
    dev = Q.device
    _row_state(O, L, D, B, Hq, N, d, dev)
    out = dict(dQt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               ddOt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               alpha=torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
               E=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    _call(dev, lib.fbob_bob_pass1, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), _p(dO), _p(UQ), _p(UK), _p(UV), _p(O), _p(L),
          _p(D), _p(out["dQt"]), _p(out["ddOt"]), _p(out["alpha"]), _p(out["E"]), _stream(dev))
    return out


def bob_pass2(Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, tau=None, causal=False):
    """Pass 2 alone (C ABI ``fbob_bob_pass2``): dKt, dVt."""
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO, UQ, UK, UV)
    dev = Q.device
    for x, name in ((L, "L"), (D, "D"), (alpha, "alpha"), (E, "E")):
        _check_f32(x, (B, Hq, N), name, dev)
    out = dict(dKt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               dVt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev))
    _call(dev, lib.fbob_bob_pass2, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), _p(dO), _p(UQ), _p(UK), _p(UV), _p(L), _p(D),
          _p(alpha), _p(E), _p(out["dKt"]), _p(out["dVt"]), _stream(dev))
    return out


def bob_workspace_size(Q, K, tau=None, causal=False) -> int:
    """Bytes of device workspace ``bob_ws`` can use for this problem (C ABI
    ``fbob_bob_workspace_size``); 0 when the problem fills the GPU unsplit."""
    lib = load_library()
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    out = ctypes.c_int64(0)
    st = lib.fbob_bob_workspace_size(_dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
                                     int(bool(causal)), ctypes.byref(out))
    if st != 0:
        raise FbobError(st)
    return int(out.value)


def bob_ws(Q, K, V, dO, UQ, UK, UV, O, L, D, tau=None, causal=False, workspace=None):
    """BoB with a caller-owned workspace (C ABI ``fbob_bob_ws``): problems too small to
    fill the GPU split their sweeps over more work-groups.  ``workspace`` is a
    contiguous GPU tensor of at least ``bob_workspace_size`` bytes (any dtype); None
    allocates one with torch.  Returns the same dict as ``bob``."""
    return _bob_ws_call("fbob_bob_ws", (), Q, K, V, dO, UQ, UK, UV, O, L, D, tau, causal,
                        workspace)


def bob_ex(Q, K, V, dO, UQ, UK, UV, O, L, D, tau=None, causal=False, flags=0, workspace=None):
    """``bob_ws`` with option bits (C ABI ``fbob_bob_ex``): ``flags`` is an OR of the
    ``FLAG_*`` values; ``FLAG_FP32_ROW_SUMS`` has Pass 1 sum alpha and E' in fp32 from
    the unrounded products (bf16 inputs at d = 64; elsewhere it changes nothing)."""
    return _bob_ws_call("fbob_bob_ex", (int(flags),), Q, K, V, dO, UQ, UK, UV, O, L, D, tau,
                        causal, workspace)


def _bob_ws_call(name, extra, Q, K, V, dO, UQ, UK, UV, O, L, D, tau, causal, workspace):
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO, UQ, UK, UV)
    dev = Q.device
    _row_state(O, L, D, B, Hq, N, d, dev)
    need = bob_workspace_size(Q, K, tau, causal)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' GPU")
    nbytes = workspace.numel() * workspace.element_size()
    out = dict(dQt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               dKt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               dVt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
               ddOt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               alpha=torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
               E=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    _call(dev, getattr(lib, name), _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), *extra,
          _p(Q), _p(K), _p(V), _p(dO), _p(UQ), _p(UK), _p(UV), _p(O), _p(L), _p(D),
          _p(out["dQt"]), _p(out["dKt"]), _p(out["dVt"]), _p(out["ddOt"]),
          _p(out["alpha"]), _p(out["E"]), _p(workspace), nbytes, _stream(dev))
    return out


def bob_noalloc(Q, K, V, dO, UQ, UK, UV, O, L, D, tau=None, causal=False, out=None):
    """BoB through the C ABI ``fbob_bob_noalloc``: the split schedule of ``bob_ws``
    with the library's static per-device scratch instead of a workspace.  ``out``
    (optional) is a dict of preallocated outputs as returned by ``bob``, so that the
    call itself allocates nothing; otherwise torch allocates them here."""
    torch = _torch()
    lib = load_library()
    B, Hq, Hkv, N, d = _check_inputs(Q, K, V, dO, UQ, UK, UV)
    dev = Q.device
    _row_state(O, L, D, B, Hq, N, d, dev)
    if out is None:
        out = dict(dQt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
                   dKt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
                   dVt=torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
                   ddOt=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
                   alpha=torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
                   E=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    shapes = dict(dQt=(B, Hq, N, d), dKt=(B, Hkv, N, d), dVt=(B, Hkv, N, d),
                  ddOt=(B, Hq, N, d), alpha=(B, Hq, N), E=(B, Hq, N))
    for k, shp in shapes.items():
        t = out[k]
        if (tuple(t.shape) != shp or t.dtype != torch.float32 or t.device != dev
                or not t.is_contiguous()):
            raise ValueError(f"out[{k!r}] must be a contiguous float32 {shp} tensor on {dev}")
    _call(dev, lib.fbob_bob_noalloc, _dtype_code(Q), B, Hq, Hkv, N, d, _tau(tau, d),
          int(bool(causal)), _p(Q), _p(K), _p(V), _p(dO), _p(UQ), _p(UK), _p(UV), _p(O), _p(L),
          _p(D), _p(out["dQt"]), _p(out["dKt"]), _p(out["dVt"]), _p(out["ddOt"]),
          _p(out["alpha"]), _p(out["E"]), _stream(dev))
    return out
