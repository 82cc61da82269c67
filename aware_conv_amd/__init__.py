"""Fused WTConv (multi-level 2-D Haar wavelet depthwise convolution) for AMD
Instinct MI355X.

The layer runs in hand-written HIP kernels behind the C ABI of
``include/wtconv.h`` (``libwtconv.so``); :mod:`aware_conv_amd._lib` binds it
with ctypes.  :class:`WTConv2d` is a drop-in replacement for a depthwise
``nn.Conv2d`` that saves only its input for the backward.

Nothing is imported eagerly, so ``import aware_conv_amd.build`` works before
the library exists.
"""

__all__ = ["WTConv2d", "WTConvFunction", "wtconv_fwd", "wtconv_bwd_input",
           "wtconv_bwd_weight", "wtconv_workspace_size"]


def __getattr__(name):
    if name in ("wtconv_fwd", "wtconv_bwd_input", "wtconv_bwd_weight",
                "wtconv_workspace_size", "wtconv_strerror", "make_shape"):
        from . import _lib
        return getattr(_lib, name)
    if name in ("WTConv2d", "WTConvFunction"):
        from . import module
        return getattr(module, name)
    raise AttributeError(name)
