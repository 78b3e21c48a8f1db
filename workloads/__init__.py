"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds NO arithmetic of the method: it only draws i.i.d. normal numbers,
scales them and rounds them to the storage type.  Both the oracle and the HIP path
consume what it returns; neither is imported here.

Recipe (one per workload, fixed order Q, K, V, dO, U_Q, U_K, U_V):
  numpy Generator(PCG64(seed)).standard_normal(shape, float32) per tensor,
  shape (B, H, N, d); optional scaling of U_* or of Q, K; then, for bf16 workloads,
  round-to-nearest-even to bfloat16 (values returned as float32 that are exactly
  representable in bf16, so both sides see identical inputs).
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np

TENSORS = ("Q", "K", "V", "dO", "UQ", "UK", "UV")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str              # "f32" or "bf16": storage type of the seven inputs
    seed: int
    scale_u: float = 1.0    # multiplies U_Q, U_K, U_V
    scale_qk: float = 1.0   # multiplies Q and K
    causal: bool = False
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def tau(self) -> float:
        """Score scale: 1/sqrt(d) unless the workload sets extra["tau"]."""
        return float(self.extra.get("tau", 1.0 / math.sqrt(self.d)))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads of the benchmark plan: sizes, dtypes, scalings and masks.
WORKLOADS = {
    "single_head_n128_d64_f32": Workload(
        "single_head_n128_d64_f32", B=1, H=1, N=128, d=64, dtype="f32", seed=1001,
        note="single head, fp32 inputs"),
    "gpt2_heads_h12_n4096_d64_bf16": Workload(
        "gpt2_heads_h12_n4096_d64_bf16", B=1, H=12, N=4096, d=64, dtype="bf16", seed=1002,
        note="GPT-2-style heads"),
    "h12_n16384_d64_bf16_u01": Workload(
        "h12_n16384_d64_bf16_u01", B=1, H=12, N=16384, d=64, dtype="bf16", seed=1003,
        scale_u=0.1, note="U_Q, U_K, U_V scaled by 0.1; headline timing workload"),
    "h8_n65536_d128_bf16_qk2": Workload(
        "h8_n65536_d128_bf16_qk2", B=1, H=8, N=65536, d=128, dtype="bf16", seed=1004,
        scale_qk=2.0, note="Q and K scaled by 2: sharp softmax rows"),
    "h1_n262144_d64_bf16": Workload(
        "h1_n262144_d64_bf16", B=1, H=1, N=262144, d=64, dtype="bf16", seed=1005,
        note="long-context single head"),
}

# The pages' isolated-op benchmark setting (FlashBoB notes, experiments table):
# causal mask, batch 4, 12 heads, bf16, at the table's sequence lengths and head dims.
for _n, _d, _seed in ((4096, 64, 2001), (8192, 64, 2002), (16384, 64, 2003),
                      (16384, 128, 2004), (32768, 128, 2005), (65536, 128, 2006),
                      (262144, 64, 2007)):
    _name = f"pages_causal_b4_h12_n{_n}_d{_d}_bf16"
    WORKLOADS[_name] = Workload(_name, B=4, H=12, N=_n, d=_d, dtype="bf16", seed=_seed,
                                causal=True, note="pages' benchmark shape (causal, B=4, H=12)")

# Grouped-query attention at the headline size (FlashBoB notes, "关键设计" 3): 12 query
# heads share 4 key/value heads (K, V, U_K, U_V keep heads 0..3 of the draw).
WORKLOADS["gqa_h12_hkv4_n16384_d64_bf16"] = Workload(
    "gqa_h12_hkv4_n16384_d64_bf16", B=1, H=12, N=16384, d=64, dtype="bf16", seed=2101,
    note="grouped-query attention, group of 3", extra={"Hkv": 4})

HEADLINE = "h12_n16384_d64_bf16_u01"


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32.

    Bit-level: add 0x7FFF plus the lowest kept bit, then clear the low 16 bits.
    Inputs here are finite normals, so NaN/Inf handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def make_inputs(w: Workload, heads=None) -> dict:
    """Draw the seven input tensors of workload ``w`` as float32 arrays (B, H, N, d).

    ``heads``: optional list of flat (b*H + h) head indices to keep; the full draw is
    still made in the fixed order so that every head's values do not depend on which
    heads are requested.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.B, w.H, w.N, w.d)
    out = {}
    for name in TENSORS:
        t = rng.standard_normal(shape, dtype=np.float32)
        if name in ("UQ", "UK", "UV") and w.scale_u != 1.0:
            t *= np.float32(w.scale_u)
        if name in ("Q", "K") and w.scale_qk != 1.0:
            t *= np.float32(w.scale_qk)
        if w.dtype == "bf16":
            t = round_to_bf16(t)
        if heads is not None:
            t = t.reshape(w.B * w.H, w.N, w.d)[list(heads)]
        out[name] = t
    return out


def make_inputs_device(w: Workload, device="cuda"):
    """The seven inputs of ``w`` drawn directly on a GPU, for lengths where a host
    draw and upload would dominate (the long-head sweep): torch's device generator
    seeded with ``w.seed``, ``randn`` in float32 per tensor in the fixed order, the
    same scalings, then rounding to the storage type (torch's float32 -> bfloat16
    conversion rounds to nearest even).  A different stream of numbers from
    ``make_inputs``; both sides of a comparison use the returned tensors.
    Returns {name: tensor [B, H, N, d]} in the storage dtype.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {}
    for name in TENSORS:
        t = torch.randn((w.B, w.H, w.N, w.d), generator=g, device=device, dtype=torch.float32)
        if name in ("UQ", "UK", "UV") and w.scale_u != 1.0:
            t *= w.scale_u
        if name in ("Q", "K") and w.scale_qk != 1.0:
            t *= w.scale_qk
        out[name] = t.to(td).contiguous()
    return out


def class_tiled(B: int, H: int, N: int, d: int, dtype: str, p: int, seed: int):
    """Inputs whose N rows are copies of p seeded "class" rows, every class used
    exactly N / p times (p must divide N), in a seeded random order.

    Returns (small, sigma): ``small`` holds the seven [B, H, p, d] float32 class
    tensors (same recipe as make_inputs: i.i.d. N(0,1), bf16-rounded for bf16), and
    ``sigma`` the length-N int64 class of each position, sigma = perm(N) mod p, so
    that the full tensor is small[..., sigma, :].  A random order (not i mod p)
    makes a row read from the wrong address land in a different class.
    """
    if N % p:
        raise ValueError("p must divide N")
    w = Workload("class_rows", B=B, H=H, N=p, d=d, dtype=dtype, seed=seed)
    small_inp = make_inputs(w)
    perm = np.random.Generator(np.random.PCG64(seed + 1)).permutation(N)
    return small_inp, (perm % p).astype(np.int64)


def small(name: str, B: int, H: int, N: int, d: int, dtype: str, seed: int,
          **kw) -> Workload:
    """An ad-hoc workload with the same recipe (used for edge-case and tail tests)."""
    return Workload(name, B=B, H=H, N=N, d=d, dtype=dtype, seed=seed, **kw)


def input_digest(inp: dict, heads) -> str:
    """SHA-256 over the float32 values of the given flat (b*H + h) heads of every
    tensor in ``inp``, tensors in draw order: identifies a seeded draw, e.g. to
    check that stored expected values were computed from the same inputs."""
    h = hashlib.sha256()
    for name in TENSORS:
        x = inp[name]
        x = x.reshape(-1, x.shape[-2], x.shape[-1])
        for f in heads:
            h.update(np.ascontiguousarray(x[f], dtype=np.float32).tobytes())
    return h.hexdigest()
