"""The oracle against an independent PyTorch-CPU float64 composition.

The composition below is written from the layer's description only: the
stride-2 analysis is torch's grouped conv2d with the printed Haar filters
(cybasar.com tutorial, section 3), each subband gets a grouped depthwise
conv2d and its scale, the synthesis is torch's conv_transpose2d with the same
filters, run from the deepest level up with the deeper reconstruction added to
the convolved LL (gist.science/pt summary, "Metodologia"), and the base path
is a depthwise conv2d with bias times its scale.  A grid with an odd side gets
one zero row (column) appended before its analysis, as TensorFlow's 'SAME'
padding does for the tutorial's stride-2 convolutions, and the transposed
convolution's output is cropped back to that grid.  Its gradients come from
torch.autograd, so the oracle's hand-written backward is checked against an
implementation it shares nothing with.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_filters():
    rows = {}
    with open(os.path.join(GOLDEN, "haar_2x2_filters.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                n, *v = line.split()
                rows[n] = [float(t) for t in v]
    return torch.tensor([rows[n] for n in ("LL", "LH", "HL", "HH")],
                        dtype=torch.float64).reshape(4, 1, 2, 2)


def torch_wtconv(x, wb, bb, sb, ww, sw):
    B, C, H, W = x.shape
    L, k = ww.shape[0], ww.shape[-1]
    dec = golden_filters().repeat(C, 1, 1, 1)  # [4C, 1, 2, 2], channel-major
    A = x
    Ys = []
    sizes = []
    for l in range(L):
        h, w = A.shape[-2:]
        sizes.append((h, w))
        S = F.conv2d(F.pad(A, (0, w % 2, 0, h % 2)), dec, stride=2, groups=C)  # [B, 4C, h', w']
        h, w = S.shape[-2:]
        A = S.view(B, C, 4, h, w)[:, :, 0]
        Y = F.conv2d(S, ww[l].reshape(4 * C, 1, k, k), padding=k // 2, groups=4 * C)
        Ys.append(Y * sw[l].reshape(1, 4 * C, 1, 1))
    R = None
    for l in reversed(range(L)):
        Y = Ys[l]
        h, w = Y.shape[-2:]
        Y5 = Y.view(B, C, 4, h, w)
        if R is not None:
            Y5 = torch.cat([(Y5[:, :, 0] + R).unsqueeze(2), Y5[:, :, 1:]], dim=2)
        R = F.conv_transpose2d(Y5.reshape(B, 4 * C, h, w), dec, stride=2, groups=C)
        R = R[:, :, :sizes[l][0], :sizes[l][1]]
    base = F.conv2d(x, wb.reshape(C, 1, k, k), bb, padding=k // 2, groups=C)
    return base * sb.reshape(1, C, 1, 1) + R


CASES = [  # B, C, H, W, L, k
    (2, 3, 16, 16, 1, 3),
    (2, 3, 16, 24, 2, 5),
    (1, 2, 32, 32, 3, 5),
    (3, 2, 32, 16, 4, 3),
    (1, 4, 64, 64, 5, 5),
    (1, 2, 28, 28, 2, 7),
    # sides not divisible by 2^L: odd grids at one or more levels
    (2, 3, 15, 13, 2, 3),
    (1, 2, 21, 10, 3, 5),
    (2, 2, 7, 9, 3, 3),
    (1, 2, 5, 5, 3, 3),
    (1, 1, 1, 3, 2, 3),
    (1, 2, 30, 30, 3, 5),
]


@pytest.mark.parametrize("B,C,H,W,L,k", CASES)
def test_forward_and_backward_match_torch(B, C, H, W, L, k):
    g = torch.Generator().manual_seed(B * 1000 + C * 100 + L * 10 + k)
    d = torch.float64
    x = torch.randn(B, C, H, W, generator=g, dtype=d)
    dy = torch.randn(B, C, H, W, generator=g, dtype=d)
    wb = (torch.randn(C, k, k, generator=g, dtype=d) * 0.2).requires_grad_()
    bb = (torch.randn(C, generator=g, dtype=d) * 0.2).requires_grad_()
    sb = (1 + 0.3 * torch.randn(C, generator=g, dtype=d)).requires_grad_()
    ww = (torch.randn(L, C, 4, k, k, generator=g, dtype=d) * 0.2).requires_grad_()
    sw = (0.5 + 0.3 * torch.randn(L, C, 4, generator=g, dtype=d)).requires_grad_()
    xr = x.clone().requires_grad_()
    y = torch_wtconv(xr, wb, bb, sb, ww, sw)
    (y * dy).sum().backward()

    args = [t.detach().numpy() for t in (wb, bb, sb, ww, sw)]
    yo = oracle.fwd(x.numpy(), *args)
    scale = y.abs().max().item()
    np.testing.assert_allclose(yo, y.detach().numpy(), rtol=0, atol=1e-12 * scale)

    go = oracle.bwd(x.numpy(), dy.numpy(), *args)
    for name, ref in [("dx", xr.grad), ("dw_base", wb.grad), ("db_base", bb.grad),
                      ("ds_base", sb.grad), ("dw_wav", ww.grad), ("ds_wav", sw.grad)]:
        ref = ref.numpy()
        np.testing.assert_allclose(go[name], ref, rtol=0,
                                   atol=1e-11 * max(1.0, np.abs(ref).max()), err_msg=name)


def test_torch_composition_gradcheck():
    """torch's autograd of the composition agrees with finite differences, so
    the composition is a sound second opinion for the backward."""
    g = torch.Generator().manual_seed(0)
    d = torch.float64
    B, C, H, W, L, k = 1, 2, 8, 8, 2, 3
    ts = [torch.randn(B, C, H, W, generator=g, dtype=d),
          torch.randn(C, k, k, generator=g, dtype=d),
          torch.randn(C, generator=g, dtype=d),
          torch.randn(C, generator=g, dtype=d),
          torch.randn(L, C, 4, k, k, generator=g, dtype=d),
          torch.randn(L, C, 4, generator=g, dtype=d)]
    ts = [t.requires_grad_() for t in ts]
    assert torch.autograd.gradcheck(torch_wtconv, ts)
