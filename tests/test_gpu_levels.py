"""Each level of the cascade checked on its own scale.

With every level in the parity cases at once, the deepest levels make up
about 1% of y and dx and a few % of the wavelet-filter gradient, so an error
in the kernels that compute only those levels would hide under the
whole-tensor bar.  Here the base scale is zero and every level but the ones
under test has zero filters: y and dx then come from those levels alone, and
every output is held to the flat bar against its own largest value (the
wavelet gradients level by level, see parity_util).  The summary of "Fast and
Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation"
(gist.science/pt, "Principais Contribuicoes") claims agreement across
decomposition levels and for all parameter gradients.

Large planes run the base conv and levels 1..3 in output tiles and the
deeper levels per plane from 8 x 8 box sums: in one workgroup's LDS while
the box sums fit (planes up to roughly 576-768 pixels a side), else level by
level through the workspace.  Whole planes run every level in one kernel.
"""
import pytest
import torch

import wtconv_inputs as wi
from parity_util import assert_parity

pytestmark = pytest.mark.gpu


def inputs(B, C, k, L, H, W, dtype, keep, seed):
    """Random per-channel scales and bias; s_base = 0 and zero filters at
    every level not in `keep` (levels counted from 1)."""
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    td = d["x"].dtype
    d["s_base"] = torch.zeros(C, dtype=td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    w = d["w_wav"].clone()
    for lv in range(1, L + 1):
        if lv not in keep:
            w[lv - 1].zero_()
    d["w_wav"] = w.contiguous()
    return d


DEEP = [  # B, C, k, L, H, W, dtype: deep levels (4..L) in one workgroup's LDS
    (2, 3, 5, 4, 256, 256, "f32"),
    (2, 3, 5, 5, 512, 512, "f32"),    # the high-resolution workload's plane
    (2, 2, 3, 6, 512, 512, "f32"),
    (1, 3, 7, 5, 256, 320, "f32"),
    (2, 3, 5, 5, 512, 512, "f16"),
    (2, 2, 5, 6, 256, 256, "f16"),
]
DEEP_DEVICE = [  # deep levels through device memory
    (2, 3, 5, 5, 1024, 1024, "f32"),
    (1, 2, 5, 4, 1024, 1024, "f32"),
    (1, 2, 7, 6, 768, 768, "f16"),
    (1, 2, 3, 5, 1024, 1024, "f16"),
    # level 1 (128²) past both staged device-memory kernels' LDS: their
    # direct forms
    (1, 1, 5, 4, 2048, 2048, "f32"),
]


@pytest.mark.parametrize("B,C,k,L,H,W,dtype", DEEP + DEEP_DEVICE)
def test_deep_levels_alone(B, C, k, L, H, W, dtype):
    """Only the levels deeper than the tile's (4..L) produce y and dx."""
    d = inputs(B, C, k, L, H, W, dtype, keep=range(4, L + 1), seed=H + W + 10 * L + k)
    assert_parity(d, dtype, "deep levels 4..%d B%d C%d k%d %dx%d %s" % (L, B, C, k, H, W, dtype))


@pytest.mark.parametrize("B,C,k,L,H,W,dtype", [
    (2, 3, 5, 5, 512, 512, "f32"),
    (1, 2, 5, 6, 1024, 1024, "f32"),
    (1, 2, 5, 6, 512, 512, "f16"),
])
def test_each_level_alone_tiles(B, C, k, L, H, W, dtype):
    """One level at a time, each of 1..L, on large planes."""
    for lv in range(1, L + 1):
        d = inputs(B, C, k, L, H, W, dtype, keep=(lv,), seed=97 * lv + H)
        assert_parity(d, dtype, "level %d of %d B%d C%d k%d %dx%d %s" % (lv, L, B, C, k, H, W,
                                                                          dtype))


@pytest.mark.parametrize("k,L,H,W,dtype", [
    (5, 6, 64, 64, "f32"), (3, 5, 32, 32, "f32"), (5, 4, 32, 32, "f16"),
    (5, 2, 56, 56, "f32"), (5, 2, 56, 56, "f16"), (5, 2, 28, 28, "f32"), (5, 1, 14, 14, "f32"),
])
def test_each_level_alone_whole_planes(k, L, H, W, dtype):
    """One level at a time on the whole-plane kernels (every level in one
    kernel), ragged batch and odd channel count."""
    for lv in range(1, L + 1):
        d = inputs(3, 5, k, L, H, W, dtype, keep=(lv,), seed=13 * lv + H + k)
        assert_parity(d, dtype, "level %d of %d k%d %dx%d %s" % (lv, L, k, H, W, dtype))
