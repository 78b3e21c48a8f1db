"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

* the library loads and exports every function declared in include/fbob.h;
* argument validation returns the documented status before any HIP call.
Pointers passed here are fake addresses: every call below is rejected (or is an
empty problem) before anything dereferences them.
"""

import ctypes
import os
import re

import pytest

from exact_softmax_attention_fbob_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fbob.h")

OK, INVALID, UNSUPPORTED, ALIGN, ALIAS, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6
SCRATCH_BYTES = 128 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fbob_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(os.path.join(ROOT, "exact_softmax_attention_fbob_amd", "libfbob.so")):
        pytest.skip("libfbob.so not built (run __graft_entry__.build())")
    return _lib.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(
        ["fbob_forward", "fbob_forward_ws", "fbob_forward_workspace_size", "fbob_backward", "fbob_backward_ws", "fbob_backward_workspace_size",
         "fbob_bob", "fbob_bob_pass1", "fbob_bob_pass2",
         "fbob_bob_workspace_size", "fbob_bob_ws", "fbob_bob_ex", "fbob_bob_noalloc",
         "fbob_strerror", "fbob_hip_error_string", "fbob_version"])
    assert sorted(_lib.PROTOTYPES) == declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.fbob_version() == 1
    for st in range(7):
        assert lib.fbob_strerror(st) != b"unknown status"
    assert lib.fbob_strerror(99) == b"unknown status"
    # no launch has failed on this thread (validation errors are not HIP errors)
    assert lib.fbob_hip_error_string() == b"no HIP error"


class FakeBuffers:
    """Disjoint, 16-byte aligned fake device addresses for every argument."""

    def __init__(self, n, stride=1 << 32):
        self.addrs = [0x100000000000 + k * stride for k in range(n)]

    def __getitem__(self, k):
        return ctypes.c_void_p(self.addrs[k])


def call_bob(lib, dtype=1, B=1, Hq=2, Hkv=2, N=64, d=64, tau=0.125, causal=0, ptrs=None):
    p = ptrs or [FakeBuffers(16)[k] for k in range(16)]
    return lib.fbob_bob(dtype, B, Hq, Hkv, N, d, ctypes.c_float(tau), causal, *p[:16],
                        ctypes.c_void_p(0))


def call_forward(lib, dtype=1, B=1, Hq=2, Hkv=2, N=64, d=64, tau=0.125, ptrs=None):
    p = ptrs or [FakeBuffers(7)[k] for k in range(7)]
    return lib.fbob_forward(dtype, B, Hq, Hkv, N, d, ctypes.c_float(tau), 0, *p[:7],
                            ctypes.c_void_p(0))


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(dtype=7), INVALID), (dict(N=-1), INVALID), (dict(B=-2), INVALID),
    (dict(Hq=3, Hkv=2), INVALID), (dict(Hkv=0), INVALID), (dict(tau=0.0), INVALID),
    (dict(tau=float("nan")), INVALID), (dict(tau=-1.0), INVALID),
    (dict(N=0), OK), (dict(B=0), OK), (dict(Hq=0, Hkv=0), OK),
    (dict(N=(1 << 31) // 64 + 1), UNSUPPORTED),
])
def test_size_validation(lib, kw, status):
    assert call_bob(lib, **kw) == status
    fkw = {k: v for k, v in kw.items() if k != "causal"}
    assert call_forward(lib, **fkw) == status


def test_null_pointer_is_invalid(lib):
    fb = FakeBuffers(16)
    for k in range(16):
        ptrs = [fb[m] for m in range(16)]
        ptrs[k] = ctypes.c_void_p(0)
        assert call_bob(lib, ptrs=ptrs) == INVALID, k


def test_misaligned_pointer(lib):
    fb = FakeBuffers(16)
    for k in range(16):
        ptrs = [fb[m] for m in range(16)]
        ptrs[k] = ctypes.c_void_p(fb.addrs[k] + 8)
        assert call_bob(lib, ptrs=ptrs) == ALIGN, k


def test_output_aliasing_an_input_or_another_output(lib):
    fb = FakeBuffers(16)
    # output dQt (index 10) placed inside input K (index 1)
    ptrs = [fb[m] for m in range(16)]
    ptrs[10] = ctypes.c_void_p(fb.addrs[1] + 16 * 64)
    assert call_bob(lib, ptrs=ptrs) == ALIAS
    # alpha (14) overlapping E (15)
    ptrs = [fb[m] for m in range(16)]
    ptrs[15] = ctypes.c_void_p(fb.addrs[14] + 16)
    assert call_bob(lib, ptrs=ptrs) == ALIAS
    # adjacent but disjoint ranges are fine up to the first launch: check with an
    # empty problem so that nothing is launched
    assert call_bob(lib, N=0, ptrs=[fb[m] for m in range(16)]) == OK


def test_pass_entry_points_validate_too(lib):
    fb = FakeBuffers(16)
    p = [fb[m] for m in range(16)]
    s = ctypes.c_void_p(0)
    assert lib.fbob_bob_pass1(1, 1, 2, 2, 64, 80, ctypes.c_float(0.1), 0, *p[:14], s) == UNSUPPORTED
    assert lib.fbob_bob_pass2(1, 1, 2, 2, 64, 80, ctypes.c_float(0.1), 0, *p[:13], s) == UNSUPPORTED
    assert lib.fbob_bob_pass1(1, 1, 2, 2, 0, 64, ctypes.c_float(0.1), 0, *p[:14], s) == OK
    q = list(p[:13])
    q[12] = ctypes.c_void_p(fb.addrs[0])  # dVt aliases Q
    assert lib.fbob_bob_pass2(1, 1, 2, 2, 64, 64, ctypes.c_float(0.1), 0, *q, s) == ALIAS


def call_backward(lib, dtype=1, B=1, Hq=2, Hkv=2, N=64, d=64, tau=0.125, causal=0, ptrs=None):
    p = ptrs or [FakeBuffers(10)[k] for k in range(10)]
    return lib.fbob_backward(dtype, B, Hq, Hkv, N, d, ctypes.c_float(tau), causal, *p[:10],
                             ctypes.c_void_p(0))


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(dtype=3), INVALID), (dict(Hq=4, Hkv=3), INVALID),
    (dict(tau=float("inf")), INVALID), (dict(N=0), OK), (dict(B=0), OK),
])
def test_backward_size_validation(lib, kw, status):
    assert call_backward(lib, **kw) == status


def test_backward_pointer_validation(lib):
    fb = FakeBuffers(10)
    for k in range(10):
        ptrs = [fb[m] for m in range(10)]
        ptrs[k] = ctypes.c_void_p(0)
        assert call_backward(lib, ptrs=ptrs) == INVALID, k
        ptrs[k] = ctypes.c_void_p(fb.addrs[k] + 4)
        assert call_backward(lib, ptrs=ptrs) == ALIGN, k
    # D (index 9) inside L (index 5); dQ (6) overlapping dK (7)
    ptrs = [fb[m] for m in range(10)]
    ptrs[9] = ctypes.c_void_p(fb.addrs[5] + 64)
    assert call_backward(lib, ptrs=ptrs) == ALIAS
    ptrs = [fb[m] for m in range(10)]
    ptrs[7] = ctypes.c_void_p(fb.addrs[6] + 1024)
    assert call_backward(lib, ptrs=ptrs) == ALIAS


def test_forward_without_do_needs_both_null(lib):
    fb = FakeBuffers(7)
    p = [fb[m] for m in range(7)]
    # dO (3) NULL with D (6) given, and the reverse: invalid
    q = list(p)
    q[3] = ctypes.c_void_p(0)
    assert call_forward(lib, ptrs=q) == INVALID
    q = list(p)
    q[6] = ctypes.c_void_p(0)
    assert call_forward(lib, ptrs=q) == INVALID
    # both NULL passes the NULL check: a misaligned Q is then what is reported
    q = list(p)
    q[3] = q[6] = ctypes.c_void_p(0)
    q[0] = ctypes.c_void_p(fb.addrs[0] + 2)
    assert call_forward(lib, ptrs=q) == ALIGN


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load_library(str(tmp_path / "libfbob.so"))


def ws_size(lib, dtype=1, B=1, Hq=12, Hkv=12, N=4096, d=64, tau=0.125, causal=0):
    out = ctypes.c_int64(-1)
    st = lib.fbob_bob_workspace_size(dtype, B, Hq, Hkv, N, d, ctypes.c_float(tau), causal,
                                     ctypes.byref(out))
    return st, out.value


def test_workspace_size_follows_the_split_plan(lib):
    """B=1 H=12 N=4096 d=64: 384 Pass 1 row tiles (1.5 rounds of 256 CUs); the first 8
    heads (256 tiles, one whole round) run unsplit and the last 4 split in two key
    parts, which fill the second round; Pass 2's 192 column tiles stay whole (four row
    parts were measured slower there: the partial sums cost more than the idle quarter
    of the CUs), so the workspace holds the 4 heads' Pass 1 partials alone.  With the
    causal mask only Pass 2 splits, at d = 64: the same shape has 96 work-groups of
    paired column tiles there, split in two.  Problems that fill the GPU, fp32 and a
    tau that is not a power of two at d = 64 need none."""
    heads, N, d = 12, 4096, 64
    assert ws_size(lib) == (OK, 2 * 4 * N * (4 * d + 2) * 4)
    # whole batches unsplit (B=3 H=4: batches 0-1, 256 tiles), the last one in two parts
    assert ws_size(lib, B=3, Hq=4, Hkv=4) == (OK, 2 * 4 * N * (4 * d + 2) * 4)
    # the leading part must not cut a group of query heads (3 per K/V head here) or a
    # batch (6 heads per batch): then every head splits, as before
    assert ws_size(lib, Hq=12, Hkv=4) == (OK, 2 * heads * N * (4 * d + 2) * 4)
    assert ws_size(lib, B=2, Hq=6, Hkv=6) == (OK, 2 * heads * N * (4 * d + 2) * 4)
    assert ws_size(lib, N=16384) == (OK, 0)            # 1536 and 768 tiles: whole rounds
    assert ws_size(lib, causal=1) == (OK, 2 * heads * N * 2 * d * 4)
    assert ws_size(lib, causal=1, B=4) == (OK, 0)      # partials would cost more
    # causal at d = 128: single tiles, split (each tile's own sweep) only while a pass's
    # tiles do not fill one round: H=12 N=4096 (384 tiles each pass) stays whole, H=4
    # (128 tiles) splits
    assert ws_size(lib, causal=1, d=128, tau=0.125) == (OK, 0)
    st, b = ws_size(lib, causal=1, d=128, tau=0.125, Hq=4, Hkv=4)
    assert st == OK and b > 0
    # B=1 H=12 N=16384: 384 Pass 2 tile pairs, 1.5 rounds; the first 8 heads fill one
    # round unsplit, the last 4 split in two parts fill the second
    assert ws_size(lib, causal=1, N=16384) == (OK, 2 * 4 * 16384 * 2 * d * 4)
    assert ws_size(lib, causal=1, N=16384, B=4) == (OK, 0)
    # B=1 H=4 N=4096: 64 Pass 1 work-groups (16 row-tile pairs x 4 heads) and 32 Pass 2
    # work-groups for 256 CUs: Pass 1 in four parts, Pass 2 in eight; the workspace
    # holds the larger of the two sets of partials (the passes reuse it in turn)
    p1 = 4 * 4 * 4096 * (4 * d + 2) * 4
    p2 = 8 * 4 * 4096 * 2 * d * 4
    assert ws_size(lib, causal=1, Hq=4, Hkv=4) == (OK, max(p1, p2))
    assert ws_size(lib, dtype=0) == (OK, 0)
    assert ws_size(lib, tau=0.1) == (OK, 0)
    # d = 128, grouped heads: Pass 2 splits the (head, row) steps of each K/V tile
    st, b = ws_size(lib, Hq=8, Hkv=2, N=8192, d=128)
    assert st == OK and b > 0
    assert ws_size(lib, N=0) == (OK, 0)
    assert ws_size(lib, d=96)[0] == UNSUPPORTED
    assert lib.fbob_bob_workspace_size(1, 1, 1, 1, 64, 64, ctypes.c_float(0.125), 0,
                                       None) == INVALID


def call_bob_ws(lib, workspace, nbytes, N=4096, Hq=12, ptrs=None):
    p = ptrs or [FakeBuffers(16)[k] for k in range(16)]
    return lib.fbob_bob_ws(1, 1, Hq, Hq, N, 64, ctypes.c_float(0.125), 0, *p[:16],
                           workspace, nbytes, ctypes.c_void_p(0))


def test_bob_ws_validates_the_workspace(lib):
    fb = FakeBuffers(17)
    ptrs = [fb[m] for m in range(16)]
    need = ws_size(lib)[1]
    assert call_bob_ws(lib, fb[16], -1, ptrs=ptrs) == INVALID
    # a workspace inside an output is an alias (checked only when it would be used)
    inside = ctypes.c_void_p(fb.addrs[10] + 1024)
    assert call_bob_ws(lib, inside, need, ptrs=ptrs) == ALIAS
    # a misaligned workspace
    assert call_bob_ws(lib, ctypes.c_void_p(fb.addrs[16] + 8), need, ptrs=ptrs) == ALIGN
    # size errors come first; the empty problem launches nothing
    assert lib.fbob_bob_ws(1, 1, 2, 2, 64, 96, ctypes.c_float(0.125), 0, *ptrs,
                           fb[16], need, ctypes.c_void_p(0)) == UNSUPPORTED
    assert call_bob_ws(lib, fb[16], need, N=0, ptrs=ptrs) == OK


def call_bob_ex(lib, flags, N=4096, d=64, ptrs=None, workspace=None, nbytes=0):
    p = ptrs or [FakeBuffers(16)[k] for k in range(16)]
    return lib.fbob_bob_ex(1, 1, 12, 12, N, d, ctypes.c_float(0.125), 0, flags, *p[:16],
                           workspace, nbytes, ctypes.c_void_p(0))


def test_bob_ex_validates_its_flags_before_any_hip_call(lib):
    """fbob_bob_ex: bits other than FBOB_FLAG_FP32_ROW_SUMS are invalid (also on an
    empty problem); size errors come first; the rest is fbob_bob_ws's validation."""
    import exact_softmax_attention_fbob_amd as fb_pkg
    text = open(HEADER).read()
    assert re.search(r"#define FBOB_FLAG_FP32_ROW_SUMS 1\b", text)
    assert fb_pkg.FLAG_FP32_ROW_SUMS == 1
    for bad in (2, 4, 3, -1, 1 << 30):
        assert call_bob_ex(lib, bad) == INVALID, bad
        assert call_bob_ex(lib, bad, N=0) == INVALID, bad
    assert call_bob_ex(lib, 1, d=96) == UNSUPPORTED
    assert call_bob_ex(lib, 1, N=0) == OK
    assert call_bob_ex(lib, 0, N=0) == OK
    fb = FakeBuffers(17)
    ptrs = [fb[m] for m in range(16)]
    ptrs[5] = ctypes.c_void_p(0)
    assert call_bob_ex(lib, 1, ptrs=ptrs) == INVALID
    ptrs = [fb[m] for m in range(16)]
    ptrs[13] = ctypes.c_void_p(fb.addrs[12] + 64)                  # ddO~ inside dV~
    assert call_bob_ex(lib, 1, ptrs=ptrs) == ALIAS
    need = ws_size(lib)[1]
    ptrs = [fb[m] for m in range(16)]
    assert call_bob_ex(lib, 1, ptrs=ptrs, workspace=fb[16], nbytes=-1) == INVALID
    assert call_bob_ex(lib, 1, ptrs=ptrs, workspace=ctypes.c_void_p(fb.addrs[16] + 8),
                       nbytes=need) == ALIGN


def test_status_names_cover_every_code(lib):
    assert sorted(_lib.STATUS) == list(range(7))
    text = open(HEADER).read()
    for code, name in _lib.STATUS.items():
        assert f"{name} = {code}" in text, name


def test_backward_workspace_size_and_validation(lib):
    """fbob_backward_workspace_size follows the first backward's split plan (B=1 H=12
    N=4096 d=64: 192 row-pass and 192 column-pass work-groups on 256 CUs); problems that
    fill the GPU, fp32 and causal problems whose tiles fill a round need none; validation
    as fbob_backward, plus the workspace's own."""
    def bws(dtype=1, B=1, Hq=12, Hkv=12, N=4096, d=64, causal=0):
        out = ctypes.c_int64(-1)
        st = lib.fbob_backward_workspace_size(dtype, B, Hq, Hkv, N, d, ctypes.c_float(0.125),
                                              causal, ctypes.byref(out))
        return st, out.value
    st, b = bws(Hq=2, Hkv=2)
    assert st == OK and b > 0
    assert bws(N=16384) == (OK, 0)
    assert bws(dtype=0, Hq=2, Hkv=2) == (OK, 0)
    assert bws(N=0) == (OK, 0)
    assert bws(d=96)[0] == UNSUPPORTED
    assert lib.fbob_backward_workspace_size(1, 1, 1, 1, 64, 64, ctypes.c_float(0.125), 0,
                                            None) == INVALID
    fb = FakeBuffers(11)
    ptrs = [fb[m] for m in range(10)]
    need = bws(Hq=2, Hkv=2)[1]

    def call(ws, nbytes, p=ptrs, N=4096):
        return lib.fbob_backward_ws(1, 1, 2, 2, N, 64, ctypes.c_float(0.125), 0, *p, ws,
                                    nbytes, ctypes.c_void_p(0))
    assert call(fb[10], -1) == INVALID
    assert call(ctypes.c_void_p(fb.addrs[6] + 64), need) == ALIAS      # inside dQ
    assert call(ctypes.c_void_p(fb.addrs[10] + 8), need) == ALIGN
    assert call(fb[10], need, N=0) == OK
    bad = list(ptrs)
    bad[2] = ctypes.c_void_p(0)
    assert call(fb[10], need, p=bad) == INVALID


def test_forward_workspace_size_and_validation(lib):
    """fbob_forward_workspace_size follows the split forward's plan: with the mask, parts =
    resident work-group slots (512 at d = 64, 256 at d = 128) over the 256-row tiles;
    without it, the part count of least estimated time (whole CU rounds x stages per part
    + the merge's traffic + a fixed cost) if that is at most 0.9 of the unsplit one; at
    most a quarter of the key stages (of the mean causal sweep) and 16; s (d + 2) fp32 per
    row.  Problems that fill the slots, fp32 ones and short sweeps need none; validation
    as fbob_forward, plus the workspace's own."""
    def fws(dtype=1, B=1, Hq=12, Hkv=12, N=4096, d=64, causal=0):
        out = ctypes.c_int64(-1)
        st = lib.fbob_forward_workspace_size(dtype, B, Hq, Hkv, N, d, ctypes.c_float(0.125),
                                             causal, ctypes.byref(out))
        return st, out.value
    rows = 12 * 4096
    assert fws() == (OK, 0)                            # 192 tiles: no split pays
    assert fws(causal=1) == (OK, 3 * rows * 66 * 4)    # mean sweep 16 stages
    assert fws(d=128) == (OK, 0)
    assert fws(Hq=2, Hkv=2) == (OK, 8 * 2 * 4096 * 66 * 4)        # 32 tiles: 8 parts
    assert fws(Hq=6, Hkv=6) == (OK, 2 * 6 * 4096 * 66 * 4)        # 96 tiles: one round
    assert fws(Hq=6, Hkv=6, d=128) == (OK, 2 * 6 * 4096 * 130 * 4)
    assert fws(Hq=2, Hkv=2, d=128) == (OK, 8 * 2 * 4096 * 130 * 4)
    assert fws(Hq=12, Hkv=12, N=8192) == (OK, 2 * 12 * 8192 * 66 * 4)  # 384 tiles
    assert fws(Hq=20, Hkv=20) == (OK, 0)
    assert fws(Hq=1, Hkv=1, N=1024) == (OK, 2 * 1024 * 66 * 4)   # 8 stages: 2 parts
    assert fws(Hq=1, Hkv=1, N=32768) == (OK, 2 * 32768 * 66 * 4)  # 128 tiles
    assert fws(Hq=1, Hkv=1, N=65536) == (OK, 0)        # 256 tiles: one round either way
    assert fws(Hq=1, Hkv=1, N=512) == (OK, 0)          # 4 stages: no split
    assert fws(N=16384) == (OK, 0)                     # 768 tiles fill 512 slots
    assert fws(dtype=0) == (OK, 0)
    assert fws(N=0) == (OK, 0)
    assert fws(d=96)[0] == UNSUPPORTED
    assert lib.fbob_forward_workspace_size(1, 1, 1, 1, 64, 64, ctypes.c_float(0.125), 0,
                                           None) == INVALID
    fb = FakeBuffers(8)
    ptrs = [fb[m] for m in range(7)]
    need = fws(Hq=2, Hkv=2)[1]
    assert need > 0

    def call(ws, nbytes, p=ptrs, N=4096):
        return lib.fbob_forward_ws(1, 1, 2, 2, N, 64, ctypes.c_float(0.125), 0, *p, ws,
                                   nbytes, ctypes.c_void_p(0))
    assert call(fb[7], -1) == INVALID
    assert call(ctypes.c_void_p(fb.addrs[4] + 64), need) == ALIAS      # inside O
    assert call(ctypes.c_void_p(fb.addrs[7] + 8), need) == ALIGN
    assert call(fb[7], need, N=0) == OK
    bad = list(ptrs)
    bad[6] = ctypes.c_void_p(0)                                         # D NULL, dO given
    assert call(fb[7], need, p=bad) == INVALID
    bad = list(ptrs)
    bad[1] = ctypes.c_void_p(0)
    assert call(fb[7], need, p=bad) == INVALID


def test_header_states_the_scratch_size():
    text = open(HEADER).read()
    assert re.search(r"#define FBOB_SCRATCH_BYTES \(\(int64_t\)128 << 20\)", text)
    assert "FBOB_ERR_SCRATCH = 6" in text


def call_bob_noalloc(lib, B=1, Hq=12, Hkv=12, N=4096, d=64, ptrs=None):
    p = ptrs or [FakeBuffers(16)[k] for k in range(16)]
    return lib.fbob_bob_noalloc(1, B, Hq, Hkv, N, d, ctypes.c_float(1 / d ** 0.5), 0, *p[:16],
                                ctypes.c_void_p(0))


def test_bob_noalloc_validates_before_any_hip_call(lib):
    """Errors that need no GPU: sizes, pointers, and a split schedule larger than the
    static scratch (B=2 H=10 N=4096 d=128: the heads of Pass 2's whole round would end
    inside a batch, so every head splits in two parts of 20 x 4096 rows x 2 x 128 fp32,
    160 MiB > 128 MiB)."""
    st, need = ws_size(lib, B=2, Hq=10, Hkv=10, N=4096, d=128, tau=1 / 128 ** 0.5)
    assert st == OK and need == 2 * 20 * 4096 * 2 * 128 * 4 > SCRATCH_BYTES
    assert call_bob_noalloc(lib, B=2, Hq=10, Hkv=10, d=128) == SCRATCH
    # the C2 problem fits (its workspace is 32.25 MiB), and so does its d = 128 form
    assert 0 < ws_size(lib)[1] <= SCRATCH_BYTES
    assert 0 < ws_size(lib, d=128, tau=1 / 128 ** 0.5)[1] <= SCRATCH_BYTES
    assert call_bob_noalloc(lib, d=96) == UNSUPPORTED
    assert call_bob_noalloc(lib, N=0) == OK
    fb = FakeBuffers(16)
    ptrs = [fb[m] for m in range(16)]
    ptrs[3] = ctypes.c_void_p(0)
    assert call_bob_noalloc(lib, B=2, Hq=10, Hkv=10, d=128, ptrs=ptrs) == INVALID  # first
    ptrs = [fb[m] for m in range(16)]
    ptrs[10] = ctypes.c_void_p(fb.addrs[0])                         # dQ~ on top of Q
    assert call_bob_noalloc(lib, B=2, Hq=10, Hkv=10, d=128, ptrs=ptrs) == ALIAS
