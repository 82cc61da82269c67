"""wtconv_bwd_noalloc (the allocation-free fused backward, whose workspace is
the library's static scratch) against wtconv_bwd on the same inputs, through
the C ABI: two calls in a row, the second on a smaller input, must give the
same bits as the workspace-taking call (same kernels, same launch)."""
import pytest
import torch

import wtconv_inputs as wi

pytestmark = pytest.mark.gpu

PARAMS = ("w_base", "b_base", "s_base", "w_wav", "s_wav")


def lib():
    from aware_conv_amd import _lib
    return _lib


def inputs(B, C, H, W, L, k, dtype, seed):
    d = {n: t.cuda() for n, t in wi.make_inputs(B, C, H, W, L, k, dtype, seed=seed).items()}
    g = torch.Generator().manual_seed(seed + 1)
    td = d["x"].dtype
    d["s_base"] = (1 + 0.5 * torch.randn(C, generator=g)).to(td).cuda()
    d["s_wav"] = (0.3 + 0.5 * torch.randn(L, C, 4, generator=g)).to(td).cuda()
    return d


def noalloc_matches_bwd(case):
    L = lib()
    d = inputs(*case, seed=sum(case[:6]))
    p = [d[n] for n in PARAMS]
    print("\ncase noalloc %s" % (case,), flush=True)
    dx_ref, g_ref = L.wtconv_bwd(d["x"], d["dy"], *p)
    dx = torch.full_like(d["x"], float("nan"))
    g = {n: torch.full_like(t, float("nan")) for n, t in zip(L.GRAD_NAMES, p)}
    L.wtconv_bwd_noalloc(d["x"], d["dy"], *p, dx, g)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref), case
    for n in L.GRAD_NAMES:
        assert torch.equal(g[n], g_ref[n]), (case, n)


@pytest.mark.parametrize("cases", [
    # whole planes: the stage-1 shape, then a smaller batch of another shape
    [(64, 96, 56, 56, 2, 5, "f32"), (3, 5, 28, 28, 2, 5, "f32")],
    # tiles with deep levels (box sums, deep contribution, partial rows in the
    # scratch), then a smaller tile shape, fp16
    [(2, 6, 512, 512, 5, 5, "f32"), (1, 3, 128, 96, 4, 3, "f16")],
    # zero-extended tiled planes (the extended tensors in the scratch), then
    # a smaller shape read as corners of whole planes
    [(4, 8, 58, 58, 2, 5, "f32"), (2, 4, 13, 13, 1, 5, "f16")],
])
def test_noalloc_twice_second_smaller(cases):
    for case in cases:
        noalloc_matches_bwd(case)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    L = lib()
    # 58 x 58 planes run on tiles, zero-extended to 60 x 60: three extended
    # tensors of 32 x 96 x 60 x 60 floats (42 MiB each) in the workspace
    d = inputs(32, 96, 58, 58, 2, 5, "f32", seed=3)
    assert L.wtconv_workspace_size(L.shape_of(d["x"], d["w_wav"])) > 64 << 20
    p = [d[n] for n in PARAMS]
    dx = torch.empty_like(d["x"])
    g = {n: torch.empty_like(t) for n, t in zip(L.GRAD_NAMES, p)}
    with pytest.raises(L.WTConvError) as e:
        L.wtconv_bwd_noalloc(d["x"], d["dy"], *p, dx, g)
    assert e.value.code == -10
