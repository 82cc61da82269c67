"""HIP path against the fp64 oracle, element by element, through the C ABI.

Error metric per output tensor: max_i |gpu_i - oracle_i| / max_i |oracle_i|
(an absolute bound where the oracle is identically zero).  Bars: 1e-5 for
fp32, 2e-2 for fp16 storage with fp32 accumulation.  For fp16 the oracle gets
the same fp16-rounded inputs, upcast to fp64.

The named workloads are run at their full sizes, in the launch configuration
the benchmark uses, and compared with the oracle on every element.  Every
case runs both backward forms: the two separate calls and the fused
wtconv_bwd, whose input gradient must equal the separate call's bit for bit
(same kernels' arithmetic in the same order).
"""
import numpy as np
import pytest
import torch

import oracle
import wtconv_inputs as wi
from parity_util import NAMES, TOL, assert_parity, lib, rel_err  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "stage1", "stage2", "stage3", "stage1_f16", "highres"])
def test_named_workload_full_size(name):
    wl = wi.WORKLOADS[name]
    print("\ncase %s %s" % (name, wl), flush=True)
    assert_parity(wi.workload_inputs(wl), wl.dtype, name)


@pytest.mark.parametrize("name", ["stage1", "stage1_f16"])
def test_wavelet_path_alone(name):
    """beta = 0 leaves only the wavelet path, so its (small) contribution is
    checked at full tolerance instead of hiding under the base conv."""
    wl = wi.WORKLOADS[name]
    d = wi.make_inputs(8, wl.C, wl.H, wl.W, wl.L, wl.k, wl.dtype, seed=3, s_base=0.0)
    assert_parity(d, wl.dtype, name + "-wavelet-only", names=("y", "dx", "dw_wav", "ds_wav", "ds_base"))


SMALL = [  # k, L, H, W: every small variant the library carries
    (1, 1, 8, 8), (3, 1, 8, 8), (3, 2, 16, 16), (3, 3, 16, 16), (5, 3, 16, 16),
    (7, 2, 16, 16), (7, 1, 14, 14), (3, 2, 16, 32), (5, 4, 32, 32), (3, 5, 32, 32),
    (5, 6, 64, 64), (5, 2, 32, 32), (5, 2, 28, 28), (5, 1, 14, 14), (5, 2, 56, 56),
    (5, 1, 8, 8), (5, 1, 56, 56), (5, 3, 56, 56), (5, 1, 28, 28), (5, 3, 32, 32),
    (5, 2, 16, 16), (5, 2, 8, 8), (5, 3, 8, 8),
]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("k,L,H,W", SMALL)
def test_small_shapes_ragged_batch(k, L, H, W, dtype):
    """Ragged batch (not a multiple of the planes per workgroup), odd channel
    count and per-channel random scales, so every index of the fold and of
    the gradient reduction is exercised."""
    B, C = 3, 5
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=k * 100 + L * 10 + H)
    g = torch.Generator().manual_seed(7)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.1 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "k%d L%d %dx%d %s" % (k, L, H, W, dtype))


TILED = [  # k, L, H, W, dtype: planes handled as tiles (+ deep levels); the
    # forward and input gradient use 32 x 64 tiles for k <= 5, the rest 32 x 32
    (3, 3, 64, 64, "f32"),    # three levels in the tile, no deep levels
    (5, 2, 48, 80, "f32"),    # partial edge tiles
    (5, 3, 40, 136, "f32"),   # two full 64-wide tiles and an 8-wide one per row
    (5, 1, 24, 72, "f16"),    # partial tiles, fp16
    (3, 2, 36, 40, "f32"),    # partial tiles, H != W
    (1, 1, 40, 40, "f32"),    # k = 1: no halo
    (5, 4, 96, 64, "f32"),    # one deep level
    (7, 5, 64, 96, "f32"),    # two deep levels, k = 7
    (5, 6, 128, 128, "f32"),  # three deep levels
    (5, 3, 64, 64, "f16"),
    (5, 5, 128, 96, "f16"),
]


@pytest.mark.parametrize("k,L,H,W,dtype", TILED)
def test_tiled_planes(k, L, H, W, dtype):
    B, C = 3, 5
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=k * 1000 + L * 100 + H + W)
    g = torch.Generator().manual_seed(11)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "tiled k%d L%d %dx%d %s" % (k, L, H, W, dtype))


@pytest.mark.parametrize("B,C,k,L,H,W,dtype", [
    (16, 7, 5, 4, 128, 192, "f32"),
    (32, 5, 5, 5, 96, 160, "f16"),
])
def test_tiled_ranges_span_images_and_channels(B, C, k, L, H, W, dtype):
    # more tiles than resident workgroups: each workgroup of the forward and
    # input gradient walks a range of tiles that runs past image and channel
    # ends, and each workgroup of the backward walks several tiles and images
    # of its channel
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=B * 100 + C)
    g = torch.Generator().manual_seed(13)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "tile ranges B%d C%d k%d L%d %dx%d %s" % (B, C, k, L, H, W, dtype))


@pytest.mark.parametrize("B,C,k,L,H,W,dtype", [
    (4, 260, 5, 2, 56, 56, "f32"),   # one-side fused backward (28-output tiles)
    (4, 260, 5, 2, 56, 56, "f16"),
    (8, 300, 5, 2, 28, 28, "f32"),   # two-side fused backward (14-output tiles)
])
def test_fused_backward_ranges_span_channels(B, C, k, L, H, W, dtype):
    """More (channel, group) items than resident workgroups, and a channel
    count of which the resident slots (three or four per compute unit on a
    256-unit device) hold no multiple within 7/8: the ranges of the fused
    backward and of the weight-only backward span channels, reducing each
    finished channel's taps on the way and folding the next channel's
    filters, in both backward kernels."""
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=C + H)
    g = torch.Generator().manual_seed(17)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.1 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "channel ranges B%d C%d k%d L%d %dx%d %s" % (B, C, k, L, H, W, dtype))


@pytest.mark.parametrize("B,C,k,L,H,W,dtype", [
    (2, 3, 5, 5, 1024, 1024, "f32"),
    (1, 2, 7, 6, 768, 768, "f16"),
    (2, 2, 3, 4, 1024, 1280, "f32"),
    (1, 2, 1, 4, 1152, 1152, "f32"),
])
def test_deep_levels_through_device_memory(B, C, k, L, H, W, dtype):
    # box sums too large for one workgroup's LDS: the deep levels run level by
    # level through the workspace (analysis, convs, synthesis, correlations)
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=H + W + L)
    g = torch.Generator().manual_seed(17)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "deep in memory B%d C%d k%d L%d %dx%d %s" % (B, C, k, L, H, W, dtype))


@pytest.mark.parametrize("B,C,k,L,H,W,dtype", [
    (3, 2, 3, 4, 512, 1536, "f32"),
    (2, 2, 1, 4, 832, 832, "f32"),
    (2, 3, 5, 5, 512, 512, "f16"),
])
def test_deep_levels_of_large_planes_in_lds(B, C, k, L, H, W, dtype):
    # the largest box sums whose deep levels still fit one workgroup's LDS
    # (one or two workgroups per compute unit): level 1 is computed from the
    # box sums in device memory, levels 2.. in LDS
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=H + W + L + 1)
    g = torch.Generator().manual_seed(23)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "deep in LDS B%d C%d k%d L%d %dx%d %s" % (B, C, k, L, H, W, dtype))


ANY_SIZE = [  # k, L, H, W, dtype: sides the kernels do not take directly
    (5, 2, 55, 55, "f32"),    # corners of 56 x 56 whole planes
    (5, 2, 27, 27, "f16"),    # of 28 x 28, fp16
    (5, 1, 13, 13, "f32"),    # of 14 x 14
    (5, 1, 7, 7, "f32"),      # ConvNeXt stage 4: of 8 x 8
    (5, 1, 7, 7, "f16"),
    (5, 3, 7, 7, "f32"),      # of the 8 x 8 three-level variant (one-side backward)
    (5, 2, 7, 7, "f16"),      # of the 8 x 8 two-level variant (two-side backward)
    (5, 1, 13, 13, "f16"),    # of 14 x 14, four planes per group, one-side backward
    (3, 3, 30, 17, "f32"),    # to 32 x 24, tiles
    (7, 2, 6, 10, "f32"),     # to 8 x 12, tiles
    (5, 3, 56, 56, "f32"),    # L = 3 at 56: divisible, tiles directly
    (5, 5, 100, 90, "f32"),   # to 128 x 96, tiles plus two deep levels
    (3, 2, 9, 7, "f16"),      # to 12 x 8, fp16 tiles
    (1, 1, 5, 3, "f32"),
    (3, 1, 1, 1, "f32"),      # one pixel: a single 1 x 1 coefficient per subband
    (5, 2, 1, 7, "f16"),      # one row: every level's grid one row high
    (7, 3, 3, 2, "f32"),      # a plane smaller than the kernel at every level
]


@pytest.mark.parametrize("H,dtype", [(7, "f32"), (8, "f32"), (7, "f16")])
def test_stage4_planes(H, dtype):
    """ConvNeXt stage-4 planes (7 x 7, read and written as corners of 8 x 8
    planes, and 8 x 8 directly) with more images than a group holds (16 planes per group) and a
    ragged last group."""
    B, C, k, L = 20, 6, 5, 1
    d = wi.make_inputs(B, C, H, H, L, k, dtype, seed=400 + H)
    g = torch.Generator().manual_seed(19)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "stage4 %dx%d %s" % (H, H, dtype))


@pytest.mark.parametrize("k,L,H,W,dtype", ANY_SIZE)
def test_any_size(k, L, H, W, dtype):
    """Odd grids at some level: the oracle pads every level's grid on its own;
    the library runs zero-extended planes and crops (whole-plane kernels
    read and write the stored corners; tiles run on extended copies)."""
    B, C = 3, 4
    d = wi.make_inputs(B, C, H, W, L, k, dtype, seed=k * 31 + L * 7 + H * 3 + W)
    g = torch.Generator().manual_seed(13)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td)
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td)
    d["b_base"] = (0.5 * torch.randn(C, generator=g)).to(td)
    assert_parity(d, dtype, "any-size k%d L%d %dx%d %s" % (k, L, H, W, dtype))


def test_single_image_single_channel():
    d = wi.make_inputs(1, 1, 56, 56, 2, 5, "f32", seed=5)
    assert_parity(d, "f32", "B1C1")


def test_outputs_fully_written_and_deterministic():
    """NaN-poisoned outputs are fully overwritten, and repeated calls give
    the same bits (fixed reduction order, no float atomics)."""
    L = lib()
    d = {k: v.cuda() for k, v in wi.make_inputs(5, 7, 28, 28, 2, 5, "f32", seed=9).items()}
    p = [d[n] for n in ("w_base", "b_base", "s_base", "w_wav", "s_wav")]
    y = torch.full_like(d["x"], float("nan"))
    L.wtconv_fwd(d["x"], *p, y=y)
    dx = torch.full_like(d["x"], float("nan"))
    L.wtconv_bwd_input(d["dy"], p[0], p[2], p[3], p[4], dx=dx)
    gr = {n: torch.full_like(t, float("nan")) for n, t in
          zip(L.GRAD_NAMES, (p[0], p[1], p[2], p[3], p[4]))}
    L.wtconv_bwd_weight(d["x"], d["dy"], *p, grads=gr)
    torch.cuda.synchronize()
    for t in [y, dx] + list(gr.values()):
        assert torch.isfinite(t).all()
    y2 = L.wtconv_fwd(d["x"], *p)
    g2 = L.wtconv_bwd_weight(d["x"], d["dy"], *p)
    dxf = torch.full_like(d["x"], float("nan"))
    gf = {n: torch.full_like(t, float("nan")) for n, t in gr.items()}
    L.wtconv_bwd(d["x"], d["dy"], *p, dx=dxf, grads=gf)
    dxf2, gf2 = L.wtconv_bwd(d["x"], d["dy"], *p)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(dxf, dx) and torch.equal(dxf2, dx)
    for n in L.GRAD_NAMES:
        assert torch.equal(gr[n], g2[n])
        assert torch.isfinite(gf[n]).all()
        assert torch.equal(gf[n], gf2[n])


def test_input_gradient_is_rotated_forward():
    """On the GPU too: bwd_input(dy) == fwd(dy) with 180-degree rotated
    kernels and zero bias."""
    L = lib()
    d = {k: v.cuda() for k, v in wi.make_inputs(4, 6, 56, 56, 2, 5, "f32", seed=2).items()}
    dx = L.wtconv_bwd_input(d["dy"], d["w_base"], d["s_base"], d["w_wav"], d["s_wav"])
    y = L.wtconv_fwd(d["dy"], d["w_base"].flip(-1, -2).contiguous(), torch.zeros_like(d["b_base"]),
                     d["s_base"], d["w_wav"].flip(-1, -2).contiguous(), d["s_wav"])
    torch.cuda.synchronize()
    assert (dx - y).abs().max().item() <= 1e-6 * y.abs().max().item()


def test_empty_batch():
    L = lib()
    d = {k: v.cuda() for k, v in wi.make_inputs(0, 4, 16, 16, 2, 3, "f32").items()}
    p = [d[n] for n in ("w_base", "b_base", "s_base", "w_wav", "s_wav")]
    y = L.wtconv_fwd(d["x"], *p)
    g = {n: torch.full_like(t, 3.0) for n, t in zip(L.GRAD_NAMES, p)}
    L.wtconv_bwd_weight(d["x"], d["dy"], *p, grads=g)
    torch.cuda.synchronize()
    assert y.shape == d["x"].shape
    for n in L.GRAD_NAMES:
        assert torch.count_nonzero(g[n]) == 0


def test_autograd_module_matches_oracle():
    from aware_conv_amd import WTConv2d
    torch.manual_seed(0)
    m = WTConv2d(8, kernel_size=5, levels=2).cuda()
    x = torch.randn(2, 8, 32, 32, device="cuda", requires_grad=True)
    dy = torch.randn(2, 8, 32, 32, device="cuda")
    y = m(x)
    y.backward(dy)
    torch.cuda.synchronize()
    p = [getattr(m, n).detach().double().cpu().numpy() for n in ("w_base", "b_base", "s_base", "w_wav", "s_wav")]
    xo = x.detach().double().cpu().numpy()
    yo = oracle.fwd(xo, *p)
    go = oracle.bwd(xo, dy.double().cpu().numpy(), *p)
    assert rel_err(y.detach().double().cpu().numpy(), yo) < 1e-5
    assert rel_err(x.grad.double().cpu().numpy(), go["dx"]) < 1e-5
    assert rel_err(m.w_wav.grad.double().cpu().numpy(), go["dw_wav"]) < 1e-5
    assert rel_err(m.s_base.grad.double().cpu().numpy(), go["ds_base"]) < 1e-5


@pytest.mark.parametrize("which", ["input", "params"])
def test_autograd_module_partial_backward(which):
    """Only the input gradient (frozen parameters) or only the parameter
    gradients (input without grad): the module takes the single call."""
    from aware_conv_amd import WTConv2d
    torch.manual_seed(1)
    m = WTConv2d(8, kernel_size=5, levels=2).cuda()
    x = torch.randn(2, 8, 32, 32, device="cuda", requires_grad=(which == "input"))
    if which == "input":
        for prm in m.parameters():
            prm.requires_grad_(False)
    dy = torch.randn(2, 8, 32, 32, device="cuda")
    m(x).backward(dy)
    torch.cuda.synchronize()
    p = [getattr(m, n).detach().double().cpu().numpy() for n in ("w_base", "b_base", "s_base", "w_wav", "s_wav")]
    go = oracle.bwd(x.detach().double().cpu().numpy(), dy.double().cpu().numpy(), *p)
    if which == "input":
        assert rel_err(x.grad.double().cpu().numpy(), go["dx"]) < 1e-5
    else:
        assert x.grad is None
        assert rel_err(m.w_base.grad.double().cpu().numpy(), go["dw_base"]) < 1e-5
        assert rel_err(m.s_wav.grad.double().cpu().numpy(), go["ds_wav"]) < 1e-5
