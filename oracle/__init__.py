"""fp64 CPU oracle of the WTConv layer (forward and backward).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or runs anything in this directory, and this directory imports nothing
from the product package.

The arithmetic lives in ``wtconv_oracle.c`` (plain C, fp64, OpenMP over the
B*C planes).  It is the literal unfused cascade of the WTConv layer as the
summary of "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
Reformulation" (gist.science/pt, "Resumo Tecnico", "Metodologia") describes
the reference implementation: Haar analysis on the raw LL, one depthwise conv
and scale per subband, the synthesis cascade from the deepest level up, and
the scaled base conv.  This module only builds the shared object and marshals
numpy arrays.

Layouts: x, y, dy, dx [B, C, H, W]; w_base [C, k, k] (a [C, 1, k, k] array
is accepted); b_base, s_base [C]; w_wav [L, C, 4, k, k]; s_wav [L, C, 4];
subband order (LL, LH, HL, HH).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wtconv_oracle.c")
# ORACLE_LIB: another build of the same oracle (the sanitized one)
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_LIB_SAN = os.path.join(_HERE, "liboracle_asan.so")
_lib = None


def build(force=False):
    """Compile wtconv_oracle.c into liboracle.so with gcc and OpenMP."""
    if os.path.exists(_LIB) and not force:
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC",
           "-o", tmp, _SRC]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def build_sanitized():
    """liboracle_asan.so: the oracle under AddressSanitizer and
    UndefinedBehaviorSanitizer (gcc), for a run of the pins with
    ORACLE_LIB pointing at it and gcc's libasan preloaded."""
    tmp = _LIB_SAN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-shared", "-fPIC",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-o", tmp, _SRC]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_SAN)
    return _LIB_SAN


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_fwd.argtypes = [i] * 6 + [dp] * 7
        lib.oracle_fwd.restype = i
        lib.oracle_bwd.argtypes = [i] * 6 + [dp] * 13
        lib.oracle_bwd.restype = i
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        lib.oracle_set_threads.argtypes = [i]
        lib.oracle_set_threads.restype = None
        lib.oracle_haar_analysis.argtypes = [i, i, dp, dp]
        lib.oracle_haar_analysis.restype = i
        lib.oracle_haar_synthesis.argtypes = [i, i, dp, dp]
        lib.oracle_haar_synthesis.restype = i
        _lib = lib
    return _lib


def num_threads():
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def set_threads(n):
    """OpenMP threads of the oracle's later calls (results do not depend on
    it: every sum runs in a fixed order within one plane or channel)."""
    _load().oracle_set_threads(int(n))


def _f64(a):
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _params(C, L, k, w_base, b_base, s_base, w_wav, s_wav):
    w_base = _f64(w_base).reshape(C, k, k)
    b_base = _f64(b_base).reshape(C)
    s_base = _f64(s_base).reshape(C)
    w_wav = _f64(w_wav).reshape(L, C, 4, k, k)
    s_wav = _f64(s_wav).reshape(L, C, 4)
    return w_base, b_base, s_base, w_wav, s_wav


def haar_analysis(z):
    """One analysis step H: z [h, w] -> subbands [4, ceil(h/2), ceil(w/2)]
    (LL, LH, HL, HH), the stride-2 2x2 Haar filtering the oracle's cascade
    uses; an odd side reads one appended zero row (column)."""
    z = _f64(z)
    h, w = z.shape
    out = np.empty((4, (h + 1) // 2, (w + 1) // 2))
    if _load().oracle_haar_analysis(h, w, _ptr(z), _ptr(out)) != 0:
        raise ValueError("bad size")
    return out


def haar_synthesis(sub, shape=None):
    """One synthesis step H^T: subbands [4, h, w] -> [2h, 2w], or cropped to
    `shape` (rows, cols), which must have ceil(rows/2) = h, ceil(cols/2) = w."""
    sub = _f64(sub)
    _, h, w = sub.shape
    rows, cols = shape if shape is not None else (2 * h, 2 * w)
    if (rows + 1) // 2 != h or (cols + 1) // 2 != w:
        raise ValueError("shape does not match the subbands")
    out = np.empty((rows, cols))
    if _load().oracle_haar_synthesis(rows, cols, _ptr(sub), _ptr(out)) != 0:
        raise ValueError("bad size")
    return out


def fwd(x, w_base, b_base, s_base, w_wav, s_wav):
    """y = WTConv(x); every array is upcast to float64 first."""
    x = _f64(x)
    B, C, H, W = x.shape
    L, k = np.asarray(w_wav).shape[0], np.asarray(w_wav).shape[-1]
    p = _params(C, L, k, w_base, b_base, s_base, w_wav, s_wav)
    y = np.empty_like(x)
    rc = _load().oracle_fwd(B, C, H, W, L, k, _ptr(x), *[_ptr(a) for a in p],
                            _ptr(y))
    if rc != 0:
        raise ValueError("oracle_fwd rejected the shape (code %d)" % rc)
    return y


def bwd(x, dy, w_base, b_base, s_base, w_wav, s_wav):
    """Gradients of <dy, WTConv(x)>.

    Returns a dict with dx [B,C,H,W], dw_base [C,k,k], db_base [C],
    ds_base [C], dw_wav [L,C,4,k,k], ds_wav [L,C,4].
    """
    x = _f64(x)
    dy = _f64(dy)
    B, C, H, W = x.shape
    L, k = np.asarray(w_wav).shape[0], np.asarray(w_wav).shape[-1]
    p = _params(C, L, k, w_base, b_base, s_base, w_wav, s_wav)
    out = {
        "dx": np.empty_like(x),
        "dw_base": np.empty((C, k, k)),
        "db_base": np.empty((C,)),
        "ds_base": np.empty((C,)),
        "dw_wav": np.empty((L, C, 4, k, k)),
        "ds_wav": np.empty((L, C, 4)),
    }
    rc = _load().oracle_bwd(
        B, C, H, W, L, k, _ptr(x), _ptr(dy), *[_ptr(a) for a in p],
        _ptr(out["dx"]), _ptr(out["dw_base"]), _ptr(out["db_base"]),
        _ptr(out["ds_base"]), _ptr(out["dw_wav"]), _ptr(out["ds_wav"]))
    if rc != 0:
        raise ValueError("oracle_bwd rejected the shape (code %d)" % rc)
    return out
