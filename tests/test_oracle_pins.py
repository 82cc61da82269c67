"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Every check here compares the oracle with something it does not share code
with: the Haar filter values printed in the cybasar.com WTConv tutorial
(section 3), the closed forms of the analysis and synthesis cascades (the
"closed-form synthesis" of the paper's "Metodologia" summary on
gist.science/pt), library routines (torch.nn.functional.conv2d, scipy's
correlate2d), exact linear-algebra identities (orthonormality, adjointness,
linearity) and finite differences.  All tests run on the CPU.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.signal import correlate2d

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SUBBANDS = ("LL", "LH", "HL", "HH")


def rand_params(C, L, k, seed=0, s_base=None, s_wav=None):
    r = np.random.default_rng(seed)
    p = {
        "w_base": r.normal(0, 0.3, (C, k, k)),
        "b_base": r.normal(0, 0.3, (C,)),
        "s_base": r.normal(1, 0.3, (C,)) if s_base is None else np.full(C, s_base),
        "w_wav": r.normal(0, 0.3, (L, C, 4, k, k)),
        "s_wav": r.normal(0.5, 0.3, (L, C, 4)) if s_wav is None else np.full((L, C, 4), s_wav),
    }
    return p


def fwd(x, p):
    return oracle.fwd(x, p["w_base"], p["b_base"], p["s_base"], p["w_wav"], p["s_wav"])


def bwd(x, dy, p):
    return oracle.bwd(x, dy, p["w_base"], p["b_base"], p["s_base"], p["w_wav"], p["s_wav"])


def sign(s, a, b):
    """Sign of tap (row bit a, column bit b) in subband s (LL, LH, HL, HH)."""
    return [1, (-1) ** b, (-1) ** a, (-1) ** (a + b)][s]


def load_golden_filters():
    rows = {}
    with open(os.path.join(GOLDEN, "haar_2x2_filters.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *vals = line.split()
            rows[name] = np.array([float(v) for v in vals]).reshape(2, 2)
    return np.stack([rows[n] for n in SUBBANDS])


# --------------------------------------------------------------------------
# Single-level Haar step
# --------------------------------------------------------------------------

def test_haar_filters_match_printed_values():
    """H applied to a unit impulse at tap (a, b) of a 2x2 block returns the
    printed filter entry of every subband at (a, b)."""
    filt = load_golden_filters()
    for a in range(2):
        for b in range(2):
            z = np.zeros((2, 2))
            z[a, b] = 1.0
            sub = oracle.haar_analysis(z)
            np.testing.assert_array_equal(sub[:, 0, 0], filt[:, a, b])


@pytest.mark.parametrize("h,w", [(5, 7), (1, 1), (3, 4), (6, 9)])
def test_haar_odd_sides_reconstruct_and_are_adjoint(h, w):
    """With one zero row (column) appended to an odd side, H is orthonormal
    on the padded grid, so the cropped H^T inverts it exactly, and the two
    maps are each other's transpose."""
    r = np.random.default_rng(h * 10 + w)
    z = r.normal(size=(h, w))
    sub = oracle.haar_analysis(z)
    assert sub.shape == (4, (h + 1) // 2, (w + 1) // 2)
    np.testing.assert_allclose(oracle.haar_synthesis(sub, (h, w)), z, rtol=0, atol=1e-14)
    s = r.normal(size=sub.shape)
    lhs = (sub * s).sum()
    rhs = (z * oracle.haar_synthesis(s, (h, w))).sum()
    assert abs(lhs - rhs) < 1e-13 * max(1.0, abs(lhs))
    # the padded tap reads zero: same subbands as analysing the padded grid
    zp = np.zeros((h + h % 2, w + w % 2))
    zp[:h, :w] = z
    np.testing.assert_array_equal(oracle.haar_analysis(zp), sub)


@pytest.mark.parametrize("H,W,L,k,extra", [(15, 13, 2, 3, 0), (21, 10, 3, 5, 0), (5, 5, 3, 3, 8),
                                           (30, 30, 3, 5, 0), (9, 14, 1, 5, 4)])
def test_padding_once_equals_padding_per_level(H, W, L, k, extra):
    """Appending zeros once, up to any multiple of 2^L, and cropping the
    result gives the per-level padded cascade: a block entirely in the padding
    has zero coefficients, so every grid is the per-level grid extended by
    zeros, and coefficients past a grid only reach outputs past the image."""
    r = np.random.default_rng(H * W + L)
    B, C = 2, 2
    x = r.normal(size=(B, C, H, W))
    dy = r.normal(size=x.shape)
    p = rand_params(C, L, k, seed=4)
    m = 1 << L
    Hp, Wp = -(-H // m) * m + extra, -(-W // m) * m + extra
    xp = np.zeros((B, C, Hp, Wp))
    xp[..., :H, :W] = x
    dyp = np.zeros_like(xp)
    dyp[..., :H, :W] = dy
    y, yp = fwd(x, p), fwd(xp, p)
    np.testing.assert_allclose(y, yp[..., :H, :W], rtol=0, atol=1e-12 * np.abs(y).max())
    g, gp = bwd(x, dy, p), bwd(xp, dyp, p)
    np.testing.assert_allclose(g["dx"], gp["dx"][..., :H, :W], rtol=0,
                               atol=1e-12 * np.abs(g["dx"]).max())
    for n in ("dw_base", "db_base", "ds_base", "dw_wav", "ds_wav"):
        np.testing.assert_allclose(g[n], gp[n], rtol=0, atol=1e-12 * np.abs(g[n]).max(), err_msg=n)


def test_haar_orthonormal_and_parseval():
    r = np.random.default_rng(1)
    z = r.normal(size=(12, 10))
    sub = oracle.haar_analysis(z)
    np.testing.assert_allclose(oracle.haar_synthesis(sub), z, atol=1e-14)
    assert abs((sub ** 2).sum() - (z ** 2).sum()) < 1e-12 * (z ** 2).sum()
    # H^T is the adjoint of H: <H z, s> = <z, H^T s>
    s = r.normal(size=sub.shape)
    assert abs((sub * s).sum() - (z * oracle.haar_synthesis(s)).sum()) < 1e-12


# --------------------------------------------------------------------------
# Independent closed forms (written here, not in the oracle)
# --------------------------------------------------------------------------

def closed_form_analysis(X, l):
    """S^l_s[i,j] = 2^-l * sum over the aligned 2^l block of sign * X, the
    sign taken from bit l-1 of the in-block offsets."""
    H, W = X.shape
    n = 1 << l
    out = np.zeros((4, H // n, W // n))
    for s in range(4):
        for i in range(H // n):
            for j in range(W // n):
                acc = 0.0
                for u in range(n):
                    for v in range(n):
                        acc += sign(s, (u >> (l - 1)) & 1, (v >> (l - 1)) & 1) * X[n * i + u, n * j + v]
                out[s, i, j] = acc / n
    return out


def closed_form_layer(X, c, p, L, k):
    """y for one plane by the closed-form analysis and the bit-indexed
    single-pass synthesis; convs by scipy's correlate2d."""
    H, W = X.shape
    y = p["s_base"][c] * (correlate2d(X, p["w_base"][c], mode="same") + p["b_base"][c])
    for l in range(1, L + 1):
        S = closed_form_analysis(X, l)
        Y = np.stack([p["s_wav"][l - 1, c, s] * correlate2d(S[s], p["w_wav"][l - 1, c, s], mode="same")
                      for s in range(4)])
        for yy in range(H):
            for xx in range(W):
                a, b = (yy >> (l - 1)) & 1, (xx >> (l - 1)) & 1
                y[yy, xx] += 2.0 ** (-l) * sum(sign(s, a, b) * Y[s, yy >> l, xx >> l] for s in range(4))
    return y


@pytest.mark.parametrize("L,k", [(1, 3), (2, 3), (2, 5), (3, 3), (3, 5)])
def test_closed_form_equals_cascade_8x8(L, k):
    r = np.random.default_rng(10 * L + k)
    B, C, H, W = 1, 2, 8, 8
    x = r.normal(size=(B, C, H, W))
    p = rand_params(C, L, k, seed=L + k)
    y = fwd(x, p)
    for c in range(C):
        ref = closed_form_layer(x[0, c], c, p, L, k)
        np.testing.assert_allclose(y[0, c], ref, rtol=0, atol=1e-13)


def test_closed_form_analysis_nonsquare():
    """The same closed form on a 16 x 8 plane (H != W) at L = 3."""
    r = np.random.default_rng(3)
    x = r.normal(size=(1, 1, 16, 8))
    p = rand_params(1, 3, 3, seed=5)
    np.testing.assert_allclose(fwd(x, p)[0, 0], closed_form_layer(x[0, 0], 0, p, 3, 3), atol=1e-13)


# --------------------------------------------------------------------------
# Special cases with a known answer
# --------------------------------------------------------------------------

def delta_kernel(k):
    d = np.zeros((k, k))
    d[k // 2, k // 2] = 1.0
    return d


@pytest.mark.parametrize("k", [1, 3, 5])
def test_level1_identity(k):
    """L = 1, every subband kernel a centred delta, gamma = 1, beta = 0:
    synthesis undoes analysis, so y = x."""
    r = np.random.default_rng(k)
    x = r.normal(size=(2, 3, 12, 10))
    C = 3
    p = rand_params(C, 1, k)
    p["s_base"] = np.zeros(C)
    p["w_wav"] = np.broadcast_to(delta_kernel(k), (1, C, 4, k, k)).copy()
    p["s_wav"] = np.ones((1, C, 4))
    np.testing.assert_allclose(fwd(x, p), x, atol=1e-14)


@pytest.mark.parametrize("k,L", [(3, 1), (5, 2), (7, 3)])
def test_zero_wavelet_weights_leave_scaled_base_conv(k, L):
    """No wavelet contribution: y = beta * (depthwise conv2d(x) + bias), the
    base conv as torch's own conv2d computes it."""
    r = np.random.default_rng(k)
    B, C, H, W = 2, 4, 16, 24
    x = r.normal(size=(B, C, H, W))
    for zero in ("weights", "scales"):
        p = rand_params(C, L, k, seed=k)
        if zero == "weights":
            p["w_wav"][:] = 0
        else:
            p["s_wav"][:] = 0
        ref = F.conv2d(torch.from_numpy(x), torch.from_numpy(p["w_base"]).reshape(C, 1, k, k),
                       torch.from_numpy(p["b_base"]), padding=k // 2, groups=C)
        ref = ref * torch.from_numpy(p["s_base"]).reshape(1, C, 1, 1)
        np.testing.assert_allclose(fwd(x, p), ref.numpy(), atol=1e-13)


@pytest.mark.parametrize("lvl", [1, 2, 3])
def test_ll_only_gives_block_mean(lvl):
    """Only the level-l LL subband with a centred delta kernel, gamma = 1,
    beta = 0: y is the mean of x over aligned 2^l x 2^l blocks."""
    L, k, C = 3, 3, 2
    r = np.random.default_rng(lvl)
    x = r.normal(size=(1, C, 16, 24))
    p = rand_params(C, L, k)
    p["s_base"] = np.zeros(C)
    p["w_wav"][:] = 0
    p["w_wav"][lvl - 1, :, 0] = delta_kernel(k)
    p["s_wav"] = np.ones((L, C, 4))
    n = 1 << lvl
    blocks = x.reshape(1, C, 16 // n, n, 24 // n, n).mean(axis=(3, 5))
    ref = np.repeat(np.repeat(blocks, n, axis=2), n, axis=3)
    np.testing.assert_allclose(fwd(x, p), ref, atol=1e-14)


def test_fold_scales_into_weights():
    """The layer with (K, gamma, Kb, bias, beta) equals the layer with the
    scales multiplied into the weights and bias and all scales 1."""
    L, k, C = 3, 5, 3
    r = np.random.default_rng(7)
    x = r.normal(size=(2, C, 16, 16))
    p = rand_params(C, L, k, seed=8)
    q = {
        "w_base": p["w_base"] * p["s_base"][:, None, None],
        "b_base": p["b_base"] * p["s_base"],
        "s_base": np.ones(C),
        "w_wav": p["w_wav"] * p["s_wav"][..., None, None],
        "s_wav": np.ones((L, C, 4)),
    }
    np.testing.assert_allclose(fwd(x, p), fwd(x, q), atol=1e-13)


def test_impulse_response_support():
    """A unit impulse reaches only the base k x k window and, per level l,
    the k*2^l-wide window of 2^l-aligned blocks around it."""
    L, k, C = 3, 3, 1
    H = W = 64
    p = rand_params(C, L, k, seed=4)
    pc = k // 2
    for (y0, x0) in [(29, 34), (32, 33), (0, 63)]:
        x = np.zeros((1, 1, H, W))
        x[0, 0, y0, x0] = 1.0
        y = (fwd(x, p) - fwd(np.zeros_like(x), p))[0, 0]  # drop beta * bias
        mask = np.zeros((H, W), bool)
        mask[max(0, y0 - pc):y0 + pc + 1, max(0, x0 - pc):x0 + pc + 1] = True
        for l in range(1, L + 1):
            n = 1 << l
            r0, c0 = ((y0 >> l) - pc) * n, ((x0 >> l) - pc) * n
            mask[max(0, r0):r0 + k * n, max(0, c0):c0 + k * n] = True
        assert np.all(y[~mask] == 0.0)
        # the deepest level's window is reached
        n = 1 << L
        r0 = ((y0 >> L) - pc) * n
        rows = [rr for rr in (max(0, r0), min(H, r0 + k * n) - 1)]
        assert any(np.abs(y[rr]).max() > 0 for rr in rows)


def test_shift_by_2L_commutes():
    """Shifting the input by a multiple of 2^L (away from the border) shifts
    the output the same way; a shift by 1 does not."""
    L, k, C = 2, 5, 2
    r = np.random.default_rng(11)
    x = np.zeros((1, C, 48, 48))
    x[:, :, 12:28, 8:30] = r.normal(size=(1, C, 16, 22))
    p = rand_params(C, L, k, seed=12)
    y = fwd(x, p)
    xs = np.roll(x, (4, 8), axis=(2, 3))
    np.testing.assert_allclose(fwd(xs, p), np.roll(y, (4, 8), axis=(2, 3)), atol=1e-14)
    x1 = np.roll(x, (1, 0), axis=(2, 3))
    assert np.abs(fwd(x1, p) - np.roll(y, (1, 0), axis=(2, 3))).max() > 1e-3


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def loss(x, p, dy):
    return float((fwd(x, p) * dy).sum())


@pytest.mark.parametrize("L,k,H,W", [(2, 3, 8, 8), (2, 5, 8, 8), (3, 3, 8, 8), (2, 3, 7, 5)])
def test_gradients_by_central_differences(L, k, H, W):
    """Every element of every gradient against the central difference of
    <dy, y>.  y is linear in x and in each parameter tensor taken alone, so
    the difference quotient is exact up to rounding for any step."""
    B, C = 2, 2
    r = np.random.default_rng(L * 10 + k)
    x = r.normal(size=(B, C, H, W))
    dy = r.normal(size=(B, C, H, W))
    p = rand_params(C, L, k, seed=3)
    g = bwd(x, dy, p)
    h = 0.5

    def check(name, arr, grad, setter):
        fd = np.zeros_like(arr)
        flat = arr.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            fp = setter(arr)
            flat[i] = old - h
            fm = setter(arr)
            flat[i] = old
            fd.reshape(-1)[i] = (fp - fm) / (2 * h)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-11 * scale, err_msg=name)

    check("dx", x.copy(), g["dx"], lambda a: loss(a, p, dy))
    for name, gname in [("w_base", "dw_base"), ("b_base", "db_base"), ("s_base", "ds_base"),
                        ("w_wav", "dw_wav"), ("s_wav", "ds_wav")]:
        arr = p[name].copy()

        def setter(a, name=name):
            q = dict(p)
            q[name] = a
            return loss(x, q, dy)
        check(name, arr, g[gname].reshape(arr.shape), setter)


def test_adjoint_dot_product():
    """<y(x) - y(0), dy> = <x, dx>: the input gradient is the transpose of
    the linear part of the layer."""
    L, k = 3, 5
    r = np.random.default_rng(5)
    x = r.normal(size=(2, 3, 32, 24))
    dy = r.normal(size=x.shape)
    p = rand_params(3, L, k, seed=9)
    lhs = ((fwd(x, p) - fwd(np.zeros_like(x), p)) * dy).sum()
    rhs = (x * bwd(x, dy, p)["dx"]).sum()
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_input_gradient_is_forward_with_rotated_kernels():
    """dx equals the forward pass applied to dy with every kernel rotated by
    180 degrees and no bias."""
    L, k, C = 2, 5, 3
    r = np.random.default_rng(6)
    x = r.normal(size=(2, C, 16, 16))
    dy = r.normal(size=x.shape)
    p = rand_params(C, L, k, seed=10)
    q = dict(p)
    q["w_base"] = p["w_base"][:, ::-1, ::-1].copy()
    q["w_wav"] = p["w_wav"][..., ::-1, ::-1].copy()
    q["b_base"] = np.zeros(C)
    np.testing.assert_allclose(bwd(x, dy, p)["dx"], fwd(dy, q), atol=1e-13)


def test_empty_batch_gives_zero_parameter_gradients():
    p = rand_params(2, 2, 3)
    x = np.zeros((0, 2, 8, 8))
    g = bwd(x, x, p)
    for n in ("dw_base", "db_base", "ds_base", "dw_wav", "ds_wav"):
        assert np.all(g[n] == 0)
    assert fwd(x, p).shape == x.shape


def test_result_independent_of_thread_count():
    """Gradient reduction order is fixed: same bits with 1 and many threads."""
    import subprocess
    import sys
    code = (
        "import sys, numpy as np; sys.path.insert(0, %r); import oracle;"
        "r=np.random.default_rng(0); x=r.normal(size=(3,2,16,16)); dy=r.normal(size=x.shape);"
        "wb=r.normal(size=(2,3,3)); bb=r.normal(size=2); sb=r.normal(size=2);"
        "ww=r.normal(size=(2,2,4,3,3)); sw=r.normal(size=(2,2,4));"
        "g=oracle.bwd(x,dy,wb,bb,sb,ww,sw); sys.stdout.write(repr(g['dw_wav'].tobytes().hex()[:4000]+g['ds_base'].tobytes().hex()))"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for t in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env))
    assert outs[0] == outs[1]


def test_set_threads_keeps_the_bits():
    """The thread count the bench's one-thread leg sets changes no result."""
    r = np.random.default_rng(1)
    x = r.normal(size=(2, 3, 16, 16))
    dy = r.normal(size=x.shape)
    p = (r.normal(size=(3, 3, 3)), r.normal(size=3), r.normal(size=3),
         r.normal(size=(2, 3, 4, 3, 3)), r.normal(size=(2, 3, 4)))
    n = oracle.num_threads()
    g0 = oracle.bwd(x, dy, *p)
    oracle.set_threads(1)
    try:
        assert oracle.num_threads() == 1
        g1 = oracle.bwd(x, dy, *p)
    finally:
        oracle.set_threads(n)
    assert oracle.num_threads() == n
    for k in g0:
        assert np.array_equal(g0[k], g1[k]), k
