"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same inputs, and compare output tensors.

Error metric per output tensor: max_i |gpu_i - oracle_i| / max_i |oracle_i|
(an absolute bound where the oracle is identically zero).  Bars: 1e-5 for
fp32, 2e-2 for fp16 storage with fp32 accumulation.  The wavelet-filter and
wavelet-scale gradients are also held to the bar level by level (each level's
slice against its own largest value), so that a deep level, whose gradients
are small next to the finer levels', is not checked only through the
finer levels' scale.
"""
import numpy as np
import torch

import oracle

TOL = {"f32": 1e-5, "f16": 2e-2}
NAMES = ("y", "dx", "dw_base", "db_base", "ds_base", "dw_wav", "ds_wav")
PARAM_NAMES = ("w_base", "b_base", "s_base", "w_wav", "s_wav")
PER_LEVEL = ("dw_wav", "ds_wav")


def lib():
    from aware_conv_amd import _lib
    return _lib


def gpu_run(d, dev="cuda", fused=False):
    L = lib()
    t = {k: v.to(dev) for k, v in d.items()}
    p = [t[n] for n in PARAM_NAMES]
    y = L.wtconv_fwd(t["x"], *p)
    if fused:
        dx, g = L.wtconv_bwd(t["x"], t["dy"], *p)
    else:
        dx = L.wtconv_bwd_input(t["dy"], p[0], p[2], p[3], p[4])
        g = L.wtconv_bwd_weight(t["x"], t["dy"], *p)
    torch.cuda.synchronize()
    out = {"y": y, "dx": dx}
    out.update(g)
    return {k: v.double().cpu().numpy() for k, v in out.items()}


def oracle_run(d):
    a = {k: v.double().numpy() for k, v in d.items()}
    p = [a[n] for n in PARAM_NAMES]
    out = {"y": oracle.fwd(a["x"], *p)}
    out.update(oracle.bwd(a["x"], a["dy"], *p))
    return out


def rel_err(g, o):
    g = g.reshape(o.shape)
    m = np.abs(o).max() if o.size else 0.0
    e = np.abs(g - o).max() if o.size else 0.0
    return e / m if m > 0 else e


def errors(g, o, names=NAMES):
    """Per-tensor errors, plus one per level of the wavelet gradients
    (keys 'dw_wav[l]', l = 1..L)."""
    errs = {n: rel_err(g[n], o[n]) for n in names}
    for n in PER_LEVEL:
        if n in names:
            ref = o[n]
            got = g[n].reshape(ref.shape)
            for lv in range(ref.shape[0]):
                errs["%s[%d]" % (n, lv + 1)] = rel_err(got[lv], ref[lv])
    return errs


def assert_parity(d, dtype, label, names=NAMES):
    """Both backward forms against the oracle; the fused call's input
    gradient must equal the separate call's bit for bit."""
    o = oracle_run(d)
    runs = {}
    for fused in (False, True):
        tag = label + (" fused" if fused else "")
        print("\ncase %s" % tag, flush=True)
        g = runs[fused] = gpu_run(d, fused=fused)
        errs = errors(g, o, names)
        print("%s: %s" % (tag, " ".join("%s=%.2e" % kv for kv in errs.items())), flush=True)
        for n in names:
            assert np.all(np.isfinite(g[n])), (tag, n)
        for n, e in errs.items():
            assert e <= TOL[dtype], (tag, n, e)
    assert np.array_equal(runs[True]["dx"], runs[False]["dx"]), label
    return o, runs
