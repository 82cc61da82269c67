"""torch.autograd and nn.Module wrappers over the C ABI."""
import torch

from . import _lib


class WTConvFunction(torch.autograd.Function):
    """Forward through ``wtconv_fwd``; backward through ``wtconv_bwd`` (input
    and parameter gradients from one pass), or the one of ``wtconv_bwd_input``
    and ``wtconv_bwd_weight`` that is needed.  Only x and the parameters are
    saved: the subband tensors are recomputed by the backward kernels."""

    @staticmethod
    def forward(ctx, x, w_base, b_base, s_base, w_wav, s_wav):
        ctx.save_for_backward(x, w_base, b_base, s_base, w_wav, s_wav)
        return _lib.wtconv_fwd(x, w_base, b_base, s_base, w_wav, s_wav)

    @staticmethod
    def backward(ctx, dy):
        x, w_base, b_base, s_base, w_wav, s_wav = ctx.saved_tensors
        dy = dy.contiguous()
        dx = None
        g = {n: None for n in _lib.GRAD_NAMES}
        want_dx, want_g = ctx.needs_input_grad[0], any(ctx.needs_input_grad[1:])
        if want_dx and want_g:
            dx, g = _lib.wtconv_bwd(x, dy, w_base, b_base, s_base, w_wav, s_wav)
        elif want_dx:
            dx = _lib.wtconv_bwd_input(dy, w_base, s_base, w_wav, s_wav)
        elif want_g:
            g = _lib.wtconv_bwd_weight(x, dy, w_base, b_base, s_base, w_wav, s_wav)
        return dx, g["dw_base"], g["db_base"], g["ds_base"], g["dw_wav"], g["ds_wav"]


class WTConv2d(torch.nn.Module):
    """Wavelet depthwise convolution with ``levels`` Haar levels and a
    ``kernel_size`` x ``kernel_size`` filter per channel and subband."""

    def __init__(self, channels, kernel_size=5, levels=2, base_scale=1.0,
                 wavelet_scale=0.1, device=None, dtype=None):
        super().__init__()
        f = {"device": device, "dtype": dtype}
        k, C, L = kernel_size, channels, levels
        self.w_base = torch.nn.Parameter(torch.empty(C, 1, k, k, **f))
        self.b_base = torch.nn.Parameter(torch.zeros(C, **f))
        self.s_base = torch.nn.Parameter(torch.full((C,), float(base_scale), **f))
        self.w_wav = torch.nn.Parameter(torch.empty(L, C, 4, k, k, **f))
        self.s_wav = torch.nn.Parameter(torch.full((L, C, 4), float(wavelet_scale), **f))
        with torch.no_grad():
            self.w_base.normal_(0, 0.02)
            self.w_wav.normal_(0, 0.02)

    def forward(self, x):
        return WTConvFunction.apply(x.contiguous(), self.w_base, self.b_base, self.s_base,
                                    self.w_wav, self.s_wav)
