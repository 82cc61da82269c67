"""Tensors of more than 2^31 elements (64-bit offsets across planes), checked
against the oracle where it stays exact at a fraction of the cost: y and dx of
one plane depend only on that plane and its channel's parameters, and a
channel's parameter gradients only on that channel's planes.

Every output keeps the fp32 bar of 1e-5.  A parameter gradient here sums
B * H * W = 34.6M products per tap: each lane adds its products over at most
64 tiles in fp32, the lanes of a workgroup meet in a fixed-order tree, and the
workgroups' partial rows are summed in fp64, so the error stays that of short
fp32 runs however long the whole sum."""
import numpy as np
import pytest
import torch

import oracle
import wtconv_inputs as wi

pytestmark = pytest.mark.gpu

PARAMS = ("w_base", "b_base", "s_base", "w_wav", "s_wav")


def rel_err(g, o):
    return np.abs(g - o).max() / max(np.abs(o).max(), 1e-30)


def channel_params(p, c):
    """The parameters of channel c as a one-channel layer (fp64 numpy)."""
    w_base, b_base, s_base, w_wav, s_wav = p
    sl = [w_base[c:c + 1], b_base[c:c + 1], s_base[c:c + 1], w_wav[:, c:c + 1], s_wav[:, c:c + 1]]
    return [t.double().cpu().numpy() for t in sl]


def test_more_than_2_31_elements():
    B, C, H, W, L, k = 33, 64, 1024, 1024, 5, 5
    n = B * C * H * W
    assert n > 2 ** 31
    free, _ = torch.cuda.mem_get_info()
    if free < 6 * n * 4:
        pytest.skip("needs %.0f GB of free device memory" % (6 * n * 4 / 1e9))
    from aware_conv_amd import _lib as lib
    d = wi.make_inputs(1, C, 32, 32, L, k, "f32", seed=3)
    g = torch.Generator().manual_seed(19)
    d["s_base"] = 1 + 0.5 * torch.randn(C, generator=g)
    d["s_wav"] = 0.3 + 0.5 * torch.randn(L, C, 4, generator=g)
    d["b_base"] = 0.5 * torch.randn(C, generator=g)
    p = [d[n_].cuda() for n_ in PARAMS]
    x, dy = wi.make_device_activations(B, C, H, W, seed=23)
    print("\ncase B%d C%d %dx%d L%d k%d (%d elements)" % (B, C, H, W, L, k, n), flush=True)
    y = lib.wtconv_fwd(x, *p)
    dx, grads = lib.wtconv_bwd(x, dy, *p)
    torch.cuda.synchronize()
    for b, c in ((0, 0), (31, 63), (17, 40)):
        xo = x[b:b + 1, c:c + 1].double().cpu().numpy()
        dyo = dy[b:b + 1, c:c + 1].double().cpu().numpy()
        po = channel_params(p, c)
        ey = rel_err(y[b:b + 1, c:c + 1].double().cpu().numpy(), oracle.fwd(xo, *po))
        edx = rel_err(dx[b:b + 1, c:c + 1].double().cpu().numpy(), oracle.bwd(xo, dyo, *po)["dx"])
        print("plane (%d, %d): y %.2e dx %.2e" % (b, c, ey, edx), flush=True)
        assert ey <= 1e-5 and edx <= 1e-5, (b, c, ey, edx)
    grad_tol = 1e-5
    for c in (0, 63):
        xo = x[:, c:c + 1].double().cpu().numpy()
        dyo = dy[:, c:c + 1].double().cpu().numpy()
        ref = oracle.bwd(xo, dyo, *channel_params(p, c))
        got = {"dw_base": grads["dw_base"][c:c + 1], "db_base": grads["db_base"][c:c + 1],
               "ds_base": grads["ds_base"][c:c + 1], "dw_wav": grads["dw_wav"][:, c:c + 1],
               "ds_wav": grads["ds_wav"][:, c:c + 1]}
        errs = {n_: rel_err(v.double().cpu().numpy().reshape(ref[n_].shape), ref[n_])
                for n_, v in got.items()}
        print("channel %d: %s" % (c, " ".join("%s=%.2e" % e for e in errs.items())), flush=True)
        for n_, e in errs.items():
            assert e <= grad_tol, (c, n_, e, grad_tol)
