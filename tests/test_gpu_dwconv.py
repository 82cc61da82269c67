"""The plain depthwise conv baseline (include/dwconv.h) against the fp64
oracle.  With every wavelet filter and scale zero and a base scale of one,
the WTConv oracle is a depthwise conv with bias (a case its own pins check
against torch's conv2d), so that configuration is the reference here:
y = conv_w(x) + bias, dx, dw = dK_b and db = dbias."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2}


def rel_err(g, o):
    g = g.reshape(o.shape)
    m = np.abs(o).max() if o.size else 0.0
    e = np.abs(g - o).max() if o.size else 0.0
    return e / m if m > 0 else e


def make(B, C, H, W, k, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    td = torch.float32 if dtype == "f32" else torch.float16
    d = {"x": torch.randn(B, C, H, W, generator=g),
         "w": 0.2 * torch.randn(C, 1, k, k, generator=g),
         "b": 0.5 * torch.randn(C, generator=g),
         "dy": torch.randn(B, C, H, W, generator=g)}
    return {n: t.to(td) for n, t in d.items()}


def oracle_ref(d, k):
    a = {n: t.double().numpy() for n, t in d.items()}
    C = a["w"].shape[0]
    zw = np.zeros((1, C, 4, k, k))
    zs = np.zeros((1, C, 4))
    one = np.ones(C)
    y = oracle.fwd(a["x"], a["w"], a["b"], one, zw, zs)
    g = oracle.bwd(a["x"], a["dy"], a["w"], a["b"], one, zw, zs)
    return {"y": y, "dx": g["dx"], "dw": g["dw_base"], "db": g["db_base"]}


CASES = [  # B, C, H, W, dtype
    (64, 96, 56, 56, "f32"),   # ConvNeXt-T stage 1
    (64, 192, 28, 28, "f32"),  # stage 2
    (64, 384, 14, 14, "f32"),  # stage 3
    (128, 96, 56, 56, "f16"),  # stage 1, fp16 storage
    (3, 5, 56, 56, "f32"),     # ragged batch, odd channel count
    (3, 5, 28, 28, "f16"),
    (5, 3, 14, 14, "f32"),
    (3, 5, 12, 20, "f32"),     # H != W
    (3, 5, 12, 20, "f16"),
]


@pytest.mark.parametrize("B,C,H,W,dtype", CASES)
def test_dwconv7_matches_oracle(B, C, H, W, dtype):
    from aware_conv_amd import _lib as L
    k = 7
    print("\ncase dwconv k7 %dx%dx%dx%d %s" % (B, C, H, W, dtype), flush=True)
    d = make(B, C, H, W, k, dtype, seed=B + C + H + W)
    t = {n: v.cuda() for n, v in d.items()}
    y = L.dwconv_fwd(t["x"], t["w"], t["b"])
    dx, dw, db = L.dwconv_bwd(t["x"], t["dy"], t["w"])
    torch.cuda.synchronize()
    got = {"y": y, "dx": dx, "dw": dw, "db": db}
    ref = oracle_ref(d, k)
    for n, r in ref.items():
        v = got[n].double().cpu().numpy()
        assert np.all(np.isfinite(v)), n
        e = rel_err(v, r)
        print("  %s %.2e" % (n, e), flush=True)
        assert e <= TOL[dtype], (n, e)


def test_dwconv_empty_batch_zero_gradients():
    from aware_conv_amd import _lib as L
    d = {n: v.cuda() for n, v in make(0, 4, 56, 56, 7, "f32", 0).items()}
    dw = torch.full_like(d["w"], 3.0)
    db = torch.full_like(d["b"], 3.0)
    L.dwconv_bwd(d["x"], d["dy"], d["w"], dw=dw, db=db)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw) == 0 and torch.count_nonzero(db) == 0
