"""Seeded synthetic inputs for the WTConv layer.

This module holds no part of the layer's arithmetic.  It is the one piece of
code that both the fp64 oracle and the HIP library's tests consume, so both
sides see bit-identical inputs.

Workloads stand in for the "WTConvNeXt configuration" the paper evaluates on
(ConvNeXt-T stage shapes with the depthwise conv replaced by WTConv, k = 5).
No dataset or trained weights are involved: every tensor is drawn from a
``torch.Generator('cpu')`` seeded with ``seed``, in the fixed order
x, w_base, b_base, w_wav, dy, with
  x, dy ~ N(0, 1);  w_base, b_base, w_wav ~ N(0, 0.02^2);
  s_base = 1.0 (base scale), s_wav = 0.1 (wavelet scales).
Everything is drawn in float32 and cast afterwards for fp16 workloads.
"""
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C: int
    H: int
    W: int
    L: int
    k: int
    dtype: str  # "f32" or "f16"

    @property
    def N(self):
        return self.B * self.C * self.H * self.W

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.float16


# Named workloads: tiny correctness case, ConvNeXt-T stage shapes, the fp16
# stage-1 shape, a high-resolution deep cascade, and the same at 1024^2 (whose
# deepest levels no longer fit one workgroup's LDS).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 32, 32, 2, 5, "f32"),
    "stage1": Workload("stage1", 64, 96, 56, 56, 2, 5, "f32"),
    "stage2": Workload("stage2", 64, 192, 28, 28, 2, 5, "f32"),
    "stage3": Workload("stage3", 64, 384, 14, 14, 1, 5, "f32"),
    "stage1_f16": Workload("stage1_f16", 128, 96, 56, 56, 2, 5, "f16"),
    "highres": Workload("highres", 8, 64, 512, 512, 5, 5, "f32"),
    "highres1024": Workload("highres1024", 8, 64, 1024, 1024, 5, 5, "f32"),
}


def make_inputs(B, C, H, W, L, k, dtype="f32", seed=0, s_base=1.0,
                s_wav=0.1, w_std=0.02, device="cpu"):
    """Return a dict of contiguous tensors in the storage dtype.

    Keys: x [B,C,H,W], w_base [C,1,k,k], b_base [C], s_base [C],
    w_wav [L,C,4,k,k], s_wav [L,C,4], dy [B,C,H,W].
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    f32 = torch.float32
    x = torch.randn((B, C, H, W), generator=g, dtype=f32)
    w_base = torch.randn((C, 1, k, k), generator=g, dtype=f32) * w_std
    b_base = torch.randn((C,), generator=g, dtype=f32) * w_std
    w_wav = torch.randn((L, C, 4, k, k), generator=g, dtype=f32) * w_std
    dy = torch.randn((B, C, H, W), generator=g, dtype=f32)
    sb = torch.full((C,), float(s_base), dtype=f32)
    sw = torch.full((L, C, 4), float(s_wav), dtype=f32)
    td = torch.float32 if dtype == "f32" else torch.float16
    out = {"x": x, "w_base": w_base, "b_base": b_base, "s_base": sb,
           "w_wav": w_wav, "s_wav": sw, "dy": dy}
    return {n: t.to(td).contiguous().to(device) for n, t in out.items()}


def make_device_activations(B, C, H, W, seed, device="cuda"):
    """x and dy ~ N(0,1) in fp32, drawn on `device` with a generator of its
    own seeded with `seed` (for tensors too large to draw on the host)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((B, C, H, W), generator=g, device=device)
    dy = torch.randn((B, C, H, W), generator=g, device=device)
    return x, dy


def workload_inputs(wl, seed=0, device="cpu", batch=None):
    """Inputs for a named workload; ``batch`` truncates B (same draws)."""
    d = make_inputs(wl.B, wl.C, wl.H, wl.W, wl.L, wl.k, wl.dtype, seed,
                    device=device)
    if batch is not None:
        d["x"] = d["x"][:batch].contiguous()
        d["dy"] = d["dy"][:batch].contiguous()
    return d
