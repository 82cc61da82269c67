"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments with the documented codes before any device call.

Runs on the CPU: every call here fails validation, which happens before the
library touches HIP, so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lb():
    from aware_conv_amd import _lib
    return _lib


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", src, re.M))
    return sorted(names)


def test_exports_every_declared_symbol(lb):
    names = declared_functions()
    assert set(names) == set(lb.EXPORTED)
    for n in names:
        assert getattr(lb.lib, n) is not None  # dlsym succeeds


def test_header_error_codes_match_binding(lb):
    src = open(os.path.join(ROOT, "include", "wtconv.h")).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"#define (WTCONV_\w+) \((-?\d+)\)", src))
    assert codes["WTCONV_ERR_UNSUPPORTED"] == -8
    for n, v in codes.items():
        assert lb.wtconv_strerror(v) not in ("", "unknown error code"), n
    assert lb.wtconv_strerror(12345) == "unknown error code"


FAKE = ctypes.c_void_p(0x100000)      # 16-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100004)        # 4-byte aligned only


# Every call below must fail validation: a call that passed would enqueue a
# kernel on fake pointers.
def fwd(lb, shape, x=FAKE, y=FAKE2, params=FAKE, ws=None, nws=0):
    return lb.lib.wtconv_fwd(ctypes.byref(shape) if shape is not None else None,
                            x, params, params, params, params, params, y, ws, nws, None)


def good(lb, **kw):
    d = dict(B=2, C=8, H=56, W=56, L=2, k=5, dtype=lb.WTCONV_F32)
    d.update(kw)
    return lb.Shape(d["B"], d["C"], d["H"], d["W"], d["L"], d["k"], d["dtype"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(H=-56), -2), (dict(H=1 << 25), -2),
    (dict(L=0), -4), (dict(L=7), -4), (dict(k=4), -3), (dict(k=9), -3), (dict(k=0), -3),
    (dict(dtype=2), -5),
    # sides that round up (to a multiple of 2^L) to no whole-plane shape run
    # on zero-extended planes in the workspace: without one the call is
    # refused
    (dict(H=58), -7), (dict(W=58), -7), (dict(H=59, W=59), -7),
])
def test_shape_errors(lb, kw, code):
    assert fwd(lb, good(lb, **kw)) == code


def test_odd_sides_need_room_for_extended_planes(lb):
    # 55 x 55 at L = 2 runs on the 56 x 56 whole-plane kernels, reading and
    # writing its planes as corners: the partial rows of 56 x 56, nothing more
    s55, s56 = good(lb, H=55, W=55), good(lb, H=56, W=56)
    assert lb.wtconv_workspace_size(s55) == lb.wtconv_workspace_size(s56)
    # 58 x 58 rounds up to 60 x 60, which only the tiles take: three extended
    # planes and the tiles' partial rows
    s58, s60 = good(lb, H=58, W=58), good(lb, H=60, W=60)
    assert lb.wtconv_workspace_size(s58) >= 3 * 2 * 8 * 60 * 60 * 4 + lb.wtconv_workspace_size(s60)


def test_null_and_alignment_errors(lb):
    s = good(lb)
    assert fwd(lb, None) == -1
    assert fwd(lb, s, x=None) == -1
    assert fwd(lb, s, params=None) == -1
    assert fwd(lb, s, x=MIS) == -6
    assert fwd(lb, s, y=MIS) == -6
    assert fwd(lb, s, params=ctypes.c_void_p(0x100001)) == -6
    assert fwd(lb, s, y=FAKE) == -9  # y aliases x


def test_bwd_input_checks(lb):
    s = good(lb)
    f = lb.lib.wtconv_bwd_input
    assert f(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE2, None, 0, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -9
    assert f(ctypes.byref(good(lb, k=2)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, None, 0, None) == -3


# Distinct, disjoint fake buffers for the backward calls: 1 GiB apart, far
# larger than any shape below, 256-byte aligned, never dereferenced.
def far(i):
    return ctypes.c_void_p((i + 1) << 30)


X, DY, DX = far(0), far(1), far(2)
PARAMS = [far(3 + i) for i in range(5)]
GRADS = [far(8 + i) for i in range(5)]
WS = far(13)


def test_bwd_weight_workspace_checks(lb):
    s = good(lb)
    need = lb.wtconv_workspace_size(s)
    assert need > 0
    f = lb.lib.wtconv_bwd_weight
    args = [ctypes.byref(s), X, DY] + PARAMS + GRADS
    assert f(*args, WS, need - 1, None) == -7
    assert f(*args, None, need, None) == -1
    assert f(*args, MIS, need, None) == -6
    bad = [ctypes.byref(s), X, DY] + PARAMS + GRADS[:4] + [None]
    assert f(*bad, WS, need, None) == -1


@pytest.mark.parametrize("fused", [False, True])
def test_gradient_buffers_must_not_alias(lb, fused):
    """Every gradient buffer against x, dy, dx, the parameters and the other
    gradients (the finalize reads the parameters while it writes the
    gradients): an overlap is refused before anything runs."""
    s = good(lb)
    need = lb.wtconv_workspace_size(s)

    def call(x=X, dy=DY, dx=DX, params=PARAMS, grads=GRADS):
        if fused:
            return lb.lib.wtconv_bwd(ctypes.byref(s), x, dy, *params, dx, *grads, WS, need - 1,
                                     None)
        return lb.lib.wtconv_bwd_weight(ctypes.byref(s), x, dy, *params, *grads, WS, need - 1,
                                        None)

    assert call() == -7  # no overlap: the checks reach the (short) workspace
    for g in range(5):
        for other in [X, DY] + PARAMS + [GR for i, GR in enumerate(GRADS) if i != g]:
            gr = list(GRADS)
            gr[g] = other
            assert call(grads=gr) == -9, (g, other)
        # a gradient that starts inside a parameter's last bytes
        gr = list(GRADS)
        gr[g] = ctypes.c_void_p(PARAMS[3].value + 2 * 8 * 4 * 25 * 4 - 4)  # last 4 bytes of w_wav
        assert call(grads=gr) == -9, g
    if fused:
        assert call(dx=GRADS[3]) == -9
        assert call(dx=PARAMS[0]) == -9
    # the empty batch writes the (zero) gradients: checked there too
    s0 = good(lb, B=0)
    gr = list(GRADS)
    gr[2] = PARAMS[2]  # ds_base over s_base
    assert lb.lib.wtconv_bwd_weight(ctypes.byref(s0), None, None, *PARAMS, *gr, None, 0,
                                    None) == -9


@pytest.mark.parametrize("call", ["fwd", "bwd_input", "bwd_weight", "bwd"])
def test_workspace_must_not_alias(lb, call):
    """The kernels write the workspace while they read the inputs and write
    the outputs: a workspace that shares a byte with any buffer of the call is
    refused before anything runs."""
    s = good(lb, H=58, W=58)  # zero-extended planes: every call uses the workspace
    need = lb.wtconv_workspace_size(s)
    assert need > 0

    def run(ws):
        if call == "fwd":
            return lb.lib.wtconv_fwd(ctypes.byref(s), X, *PARAMS, DX, ws, need, None)
        if call == "bwd_input":
            p = [PARAMS[0], PARAMS[2], PARAMS[3], PARAMS[4]]
            return lb.lib.wtconv_bwd_input(ctypes.byref(s), DY, *p, DX, ws, need, None)
        if call == "bwd_weight":
            return lb.lib.wtconv_bwd_weight(ctypes.byref(s), X, DY, *PARAMS, *GRADS, ws, need,
                                            None)
        return lb.lib.wtconv_bwd(ctypes.byref(s), X, DY, *PARAMS, DX, *GRADS, ws, need, None)

    bufs = {"fwd": [X, DX] + PARAMS, "bwd_input": [DY, DX, PARAMS[0]] + PARAMS[2:],
            "bwd_weight": [X, DY] + PARAMS + GRADS, "bwd": [X, DY, DX] + PARAMS + GRADS}[call]
    for b in bufs:
        assert run(b) == -9, b
        # a workspace that ends inside the buffer
        assert run(ctypes.c_void_p(b.value - need + 16)) == -9, b


def test_workspace_size_queries(lb):
    n = ctypes.c_size_t(7)
    huge = good(lb, H=32768, W=32768, L=4)  # 4 GiB planes: beyond 32-bit plane offsets
    assert lb.lib.wtconv_workspace_size(ctypes.byref(huge), ctypes.byref(n)) == -8
    assert n.value == 7  # untouched on error
    assert lb.lib.wtconv_workspace_size(ctypes.byref(good(lb)), None) == -1
    assert lb.wtconv_workspace_size(good(lb, B=0)) == 0
    # grows with the batch, fixed per shape
    assert lb.wtconv_workspace_size(good(lb, B=64)) >= lb.wtconv_workspace_size(good(lb, B=2))
    assert lb.wtconv_workspace_size(good(lb, B=64)) == lb.wtconv_workspace_size(good(lb, B=64))


def test_empty_tensors_need_no_pointers(lb):
    # B = 0: nothing to compute, nothing dereferenced, no launch
    s = good(lb, B=0)
    assert fwd(lb, s, x=None, y=None) == 0
    s = good(lb, C=0)
    assert fwd(lb, s, x=None, y=None, params=None) == 0


def test_fused_bwd_checks(lb):
    s = good(lb)
    need = lb.wtconv_workspace_size(s)
    f = lb.lib.wtconv_bwd

    def call(shape=s, x=X, dy=DY, dx=DX, ws=WS, nws=need - 1, grads=GRADS):
        return f(ctypes.byref(shape), x, dy, *PARAMS, dx, *grads, ws, nws, None)

    assert call() == -7                     # workspace one byte short
    assert call(nws=need, ws=None) == -1
    assert call(dx=None) == -1
    assert call(grads=[None] * 5) == -1
    assert call(dx=MIS) == -6
    assert call(dx=X) == -9                 # dx aliases x
    assert call(dx=DY) == -9                # dx aliases dy
    assert call(shape=good(lb, k=2)) == -3
    big = [ctypes.c_void_p(n << 40) for n in (1, 2, 3)]  # 1 TiB apart: no overlap
    assert call(shape=good(lb, H=32768, W=32768, L=4), x=big[0], dy=big[1], dx=big[2]) == -8


def test_noalloc_bwd_checks(lb):
    """The allocation-free fused backward runs the same checks as wtconv_bwd,
    then refuses shapes whose workspace exceeds its static scratch, all
    before touching the device."""
    f = lb.lib.wtconv_bwd_noalloc

    def call(shape, x=X, dy=DY, dx=DX, grads=GRADS):
        return f(ctypes.byref(shape), x, dy, *PARAMS, dx, *grads, None)

    assert f(None, X, DY, *PARAMS, DX, *GRADS, None) == -1
    assert call(good(lb, k=4)) == -3
    assert call(good(lb), dx=None) == -1
    assert call(good(lb), dx=MIS) == -6
    assert call(good(lb), dx=DY) == -9
    assert call(good(lb), grads=GRADS[:4] + [PARAMS[4]]) == -9
    limit = 64 << 20
    src = open(os.path.join(ROOT, "include", "wtconv.h")).read()
    assert "#define WTCONV_NOALLOC_SCRATCH_BYTES (64u << 20)" in src
    # 8 x 64 x 1024^2 at five levels needs ~225 MiB: refused
    s = good(lb, B=8, C=64, H=1024, W=1024, L=5)
    assert lb.wtconv_workspace_size(s) > limit
    big = [ctypes.c_void_p(n << 40) for n in (1, 2, 3)]  # 1 TiB apart: 2 GiB tensors
    assert call(s, x=big[0], dy=big[1], dx=big[2]) == -10
    # the named stage shapes fit (a few MiB); 8 x 64 x 512^2 at five levels too
    for kw in (dict(B=64, C=96, H=56, W=56), dict(B=64, C=384, H=14, W=14, L=1),
               dict(B=8, C=64, H=512, W=512, L=5)):
        assert lb.wtconv_workspace_size(good(lb, **kw)) <= limit, kw


def test_dwconv_checks(lb):
    s = lb.DwShape(2, 8, 56, 56, 7, lb.WTCONV_F32)
    f, b = lb.lib.dwconv_fwd, lb.lib.dwconv_bwd
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None) == -9      # y aliases x
    assert f(ctypes.byref(s), None, FAKE, FAKE, FAKE2, None) == -1
    assert f(ctypes.byref(s), MIS, FAKE, FAKE, FAKE2, None) == -6
    assert f(ctypes.byref(lb.DwShape(2, 8, 56, 56, 6, 0)), FAKE, FAKE, FAKE, FAKE2, None) == -3
    assert f(ctypes.byref(lb.DwShape(2, 8, 57, 56, 7, 0)), FAKE, FAKE, FAKE, FAKE2, None) == -8
    assert f(ctypes.byref(lb.DwShape(-1, 8, 56, 56, 7, 0)), FAKE, FAKE, FAKE, FAKE2, None) == -2
    need = lb.dwconv_workspace_size(s)
    assert need > 0
    DX = ctypes.c_void_p(0x300000)
    assert b(ctypes.byref(s), FAKE, FAKE2, FAKE, DX, FAKE, FAKE, FAKE, need - 1, None) == -7
    assert b(ctypes.byref(s), FAKE, FAKE2, FAKE, FAKE2, FAKE, FAKE, FAKE, need, None) == -9
    assert b(ctypes.byref(s), FAKE, FAKE2, FAKE, None, FAKE, FAKE, FAKE, need, None) == -1


def test_huge_channel_counts_leave_the_whole_plane_path(lb):
    # a group's buffer offsets are 32-bit: with 2^22 channels of 56 x 56 the
    # library still sizes a workspace (the tile path takes the shape)
    s = good(lb, B=1, C=1 << 22)
    assert lb.wtconv_workspace_size(s) > 0


def test_large_planes_with_deep_levels_are_supported(lb):
    # box sums too large for one workgroup's LDS: the deep levels run through
    # device memory, which the workspace holds (three level sets of the box
    # sums on top of the partial rows, D and both box sums)
    for H, W, L, k in ((8192, 8192, 4, 5), (1024, 1024, 5, 5), (768, 768, 6, 7)):
        s = good(lb, B=1, C=2, H=H, W=W, L=L, k=k)
        p = 2 * (H >> 3) * (W >> 3) * 4  # bytes of one box-sum tensor
        levels = 4 * p * (1 - 4.0 ** -(L - 3)) / 3  # levels 4..L of one box-sum tensor
        assert lb.wtconv_workspace_size(s) >= 3 * p + 3 * levels

