"""ctypes binding of libwtconv.so (the C ABI declared in include/wtconv.h).

Argument marshalling only: shapes are read from the tensors, outputs and the
workspace are allocated with torch (device memory and streams are all torch is
used for here), and every step of the layer runs in the library's HIP kernels.
There is no fallback: if the shared object is missing, importing this module
raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# WTCONV_LIB: another build of the same library (the host-sanitized
# libwtconv_asan.so for the CPU ABI tests)
LIB_PATH = os.environ.get("WTCONV_LIB") or os.path.join(_HERE, "libwtconv.so")

WTCONV_F32 = 0
WTCONV_F16 = 1
MAX_LEVELS = 6

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libwtconv.so is not built (%s); run `python -m aware_conv_amd.build` "
        "or __graft_entry__.build() first" % LIB_PATH)


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int),
                ("W", ctypes.c_int), ("L", ctypes.c_int), ("k", ctypes.c_int),
                ("dtype", ctypes.c_int)]


class DwShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int),
                ("W", ctypes.c_int), ("k", ctypes.c_int), ("dtype", ctypes.c_int)]


lib = ctypes.CDLL(LIB_PATH)
_vp = ctypes.c_void_p
_sp = ctypes.POINTER(Shape)
lib.wtconv_workspace_size.argtypes = [_sp, ctypes.POINTER(ctypes.c_size_t)]
lib.wtconv_workspace_size.restype = ctypes.c_int
lib.wtconv_fwd.argtypes = [_sp] + [_vp] * 7 + [_vp, ctypes.c_size_t, _vp]
lib.wtconv_fwd.restype = ctypes.c_int
lib.wtconv_bwd_input.argtypes = [_sp] + [_vp] * 6 + [_vp, ctypes.c_size_t, _vp]
lib.wtconv_bwd_input.restype = ctypes.c_int
lib.wtconv_bwd_weight.argtypes = [_sp] + [_vp] * 12 + [_vp, ctypes.c_size_t, _vp]
lib.wtconv_bwd_weight.restype = ctypes.c_int
lib.wtconv_bwd.argtypes = [_sp] + [_vp] * 13 + [_vp, ctypes.c_size_t, _vp]
lib.wtconv_bwd.restype = ctypes.c_int
lib.wtconv_bwd_noalloc.argtypes = [_sp] + [_vp] * 13 + [_vp]
lib.wtconv_bwd_noalloc.restype = ctypes.c_int
_dp = ctypes.POINTER(DwShape)
lib.dwconv_workspace_size.argtypes = [_dp, ctypes.POINTER(ctypes.c_size_t)]
lib.dwconv_workspace_size.restype = ctypes.c_int
lib.dwconv_fwd.argtypes = [_dp] + [_vp] * 5
lib.dwconv_fwd.restype = ctypes.c_int
lib.dwconv_bwd.argtypes = [_dp] + [_vp] * 7 + [ctypes.c_size_t, _vp]
lib.dwconv_bwd.restype = ctypes.c_int
lib.wtconv_strerror.argtypes = [ctypes.c_int]
lib.wtconv_strerror.restype = ctypes.c_char_p

EXPORTED = ("wtconv_workspace_size", "wtconv_fwd", "wtconv_bwd_input",
            "wtconv_bwd_weight", "wtconv_bwd", "wtconv_bwd_noalloc", "wtconv_strerror",
            "dwconv_workspace_size", "dwconv_fwd", "dwconv_bwd")


class WTConvError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, wtconv_strerror(code), code))


def wtconv_strerror(code):
    return lib.wtconv_strerror(int(code)).decode()


def _dtype_code(dt):
    if dt == torch.float32:
        return WTCONV_F32
    if dt == torch.float16:
        return WTCONV_F16
    raise TypeError("WTConv supports float32 and float16 tensors, got %s" % dt)


def make_shape(B, C, H, W, L, k, dtype):
    """dtype: a torch dtype or a WTCONV_* code."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return Shape(int(B), int(C), int(H), int(W), int(L), int(k), int(code))


def shape_of(x, w_wav):
    B, C, H, W = x.shape
    return make_shape(B, C, H, W, w_wav.shape[0], w_wav.shape[-1], x.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _layer_dims(x, w_wav):
    """(B, C, H, W, L, k) from the activation and the wavelet filters."""
    if x.dim() != 4:
        raise ValueError("activations must be 4-D [B, C, H, W], got shape %s" % (tuple(x.shape),))
    if w_wav.dim() != 5 or w_wav.shape[2] != 4 or w_wav.shape[3] != w_wav.shape[4]:
        raise ValueError("w_wav must be [L, C, 4, k, k], got shape %s" % (tuple(w_wav.shape),))
    B, C, H, W = x.shape
    return B, C, H, W, w_wav.shape[0], w_wav.shape[-1]


def _expect(dtype, tensors):
    """Every (name, tensor, shape) of `tensors` (tensor None: skipped; the
    library reports a missing pointer): of that shape, of `dtype` (None: any)
    and contiguous.  The library sees only pointers and sizes, so a tensor of
    another shape would be read out of its bounds."""
    for name, t, shape in tensors:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if dtype is not None and t.dtype != dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _on_gpu(x, tensors):
    """x on a GPU and every other tensor on the same one (checked after the
    shapes, which do not depend on the device)."""
    if x.device.type != "cuda":
        raise ValueError("x is on %s; every tensor must be on a GPU" % x.device)
    for name, t in tensors:
        if t is not None and t.device != x.device:
            raise ValueError("%s is on %s; every tensor must be on %s" % (name, t.device, x.device))


def _param_specs(C, L, k, w_base, b_base, s_base, w_wav, s_wav):
    return [("w_base", w_base, (C, 1, k, k)), ("b_base", b_base, (C,)),
            ("s_base", s_base, (C,)), ("w_wav", w_wav, (L, C, 4, k, k)),
            ("s_wav", s_wav, (L, C, 4))]


def _check_call(x, w_wav, acts, params, workspace):
    """Shared checks: the activations `acts` ([B, C, H, W] each), the
    parameters, and the workspace (any dtype)."""
    B, C, H, W, L, k = _layer_dims(x, w_wav)
    specs = [(n, t, (B, C, H, W)) for n, t in acts] + _param_specs(C, L, k, *params)
    _expect(x.dtype, specs)
    _expect(None, [("workspace", workspace, None)])
    _on_gpu(x, [(n, t) for n, t, _ in specs] + [("workspace", workspace)])


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, where):
    if rc != 0:
        raise WTConvError(rc, where)


def wtconv_workspace_size(shape):
    n = ctypes.c_size_t(0)
    _check(lib.wtconv_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "wtconv_workspace_size")
    return int(n.value)


def _workspace(shape, device, workspace):
    need = wtconv_workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def wtconv_fwd(x, w_base, b_base, s_base, w_wav, s_wav, y=None,
               workspace=None, stream=None):
    """y = WTConv(x) on x's device; returns y."""
    _check_call(x, w_wav, [("x", x), ("y", y)], (w_base, b_base, s_base, w_wav, s_wav),
                workspace)
    s = shape_of(x, w_wav)
    if y is None:
        y = torch.empty_like(x)
    ws, nws = _workspace(s, x.device, workspace)
    _check(lib.wtconv_fwd(ctypes.byref(s), _ptr(x), _ptr(w_base), _ptr(b_base),
                          _ptr(s_base), _ptr(w_wav), _ptr(s_wav), _ptr(y),
                          _ptr(ws), nws, _stream(stream, x.device)), "wtconv_fwd")
    return y


def wtconv_bwd_input(dy, w_base, s_base, w_wav, s_wav, dx=None,
                     workspace=None, stream=None):
    """dx = transpose of the layer applied to dy; returns dx."""
    _check_call(dy, w_wav, [("dy", dy), ("dx", dx)], (w_base, None, s_base, w_wav, s_wav),
                workspace)
    s = shape_of(dy, w_wav)
    if dx is None:
        dx = torch.empty_like(dy)
    ws, nws = _workspace(s, dy.device, workspace)
    _check(lib.wtconv_bwd_input(ctypes.byref(s), _ptr(dy), _ptr(w_base),
                                _ptr(s_base), _ptr(w_wav), _ptr(s_wav), _ptr(dx),
                                _ptr(ws), nws, _stream(stream, dy.device)),
           "wtconv_bwd_input")
    return dx


GRAD_NAMES = ("dw_base", "db_base", "ds_base", "dw_wav", "ds_wav")


def _grads(w_base, b_base, s_base, w_wav, s_wav):
    return {"dw_base": torch.empty_like(w_base), "db_base": torch.empty_like(b_base),
            "ds_base": torch.empty_like(s_base), "dw_wav": torch.empty_like(w_wav),
            "ds_wav": torch.empty_like(s_wav)}


def _check_grads(x, w_wav, grads):
    if grads is None:
        return
    B, C, H, W, L, k = _layer_dims(x, w_wav)
    missing = [n for n in GRAD_NAMES if n not in grads]
    if missing:
        raise KeyError("grads lacks %s" % ", ".join(missing))
    specs = [("grads[%s]" % g, t, sh) for g, (_, t, sh) in
             zip(GRAD_NAMES, _param_specs(C, L, k, *[grads[n] for n in GRAD_NAMES]))]
    _expect(x.dtype, specs)


def _grads_on_gpu(x, grads):
    if grads is not None:
        _on_gpu(x, [("grads[%s]" % n, grads[n]) for n in GRAD_NAMES])


def wtconv_bwd_weight(x, dy, w_base, b_base, s_base, w_wav, s_wav, grads=None,
                      workspace=None, stream=None):
    """Parameter gradients; returns a dict keyed by GRAD_NAMES."""
    _check_grads(x, w_wav, grads)
    _check_call(x, w_wav, [("x", x), ("dy", dy)], (w_base, b_base, s_base, w_wav, s_wav),
                workspace)
    _grads_on_gpu(x, grads)
    s = shape_of(x, w_wav)
    if grads is None:
        grads = _grads(w_base, b_base, s_base, w_wav, s_wav)
    ws, nws = _workspace(s, x.device, workspace)
    _check(lib.wtconv_bwd_weight(
        ctypes.byref(s), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(b_base), _ptr(s_base),
        _ptr(w_wav), _ptr(s_wav), *[_ptr(grads[n]) for n in GRAD_NAMES],
        _ptr(ws), nws, _stream(stream, x.device)), "wtconv_bwd_weight")
    return grads


def wtconv_bwd(x, dy, w_base, b_base, s_base, w_wav, s_wav, dx=None, grads=None,
               workspace=None, stream=None):
    """Input and parameter gradients in one call; returns (dx, grads dict)."""
    _check_grads(x, w_wav, grads)
    _check_call(x, w_wav, [("x", x), ("dy", dy), ("dx", dx)],
                (w_base, b_base, s_base, w_wav, s_wav), workspace)
    _grads_on_gpu(x, grads)
    s = shape_of(x, w_wav)
    if dx is None:
        dx = torch.empty_like(dy)
    if grads is None:
        grads = _grads(w_base, b_base, s_base, w_wav, s_wav)
    ws, nws = _workspace(s, x.device, workspace)
    _check(lib.wtconv_bwd(
        ctypes.byref(s), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(b_base), _ptr(s_base),
        _ptr(w_wav), _ptr(s_wav), _ptr(dx), *[_ptr(grads[n]) for n in GRAD_NAMES],
        _ptr(ws), nws, _stream(stream, x.device)), "wtconv_bwd")
    return dx, grads


def wtconv_bwd_noalloc(x, dy, w_base, b_base, s_base, w_wav, s_wav, dx, grads,
                       stream=None):
    """wtconv_bwd with the library's static scratch as its workspace: the
    outputs dx and grads (a dict keyed by GRAD_NAMES) are the caller's, and
    nothing is allocated, here or in the library.  Returns (dx, grads)."""
    if dx is None or grads is None:
        raise ValueError("wtconv_bwd_noalloc writes into caller-provided dx and grads")
    _check_grads(x, w_wav, grads)
    _check_call(x, w_wav, [("x", x), ("dy", dy), ("dx", dx)],
                (w_base, b_base, s_base, w_wav, s_wav), None)
    _grads_on_gpu(x, grads)
    s = shape_of(x, w_wav)
    _check(lib.wtconv_bwd_noalloc(
        ctypes.byref(s), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(b_base), _ptr(s_base),
        _ptr(w_wav), _ptr(s_wav), _ptr(dx), *[_ptr(grads[n]) for n in GRAD_NAMES],
        _stream(stream, x.device)), "wtconv_bwd_noalloc")
    return dx, grads


# ---------------------------------------------------------------------------
# Plain depthwise conv baseline (include/dwconv.h)
# ---------------------------------------------------------------------------

def dw_shape_of(x, w):
    B, C, H, W = x.shape
    return DwShape(int(B), int(C), int(H), int(W), int(w.shape[-1]), _dtype_code(x.dtype))


def _check_dw(x, w, acts, others):
    if x.dim() != 4:
        raise ValueError("activations must be 4-D [B, C, H, W], got shape %s" % (tuple(x.shape),))
    if w.dim() != 4 or w.shape[1] != 1 or w.shape[2] != w.shape[3]:
        raise ValueError("w must be [C, 1, k, k], got shape %s" % (tuple(w.shape),))
    B, C, H, W = x.shape
    k = w.shape[-1]
    specs = ([(n, t, (B, C, H, W)) for n, t in acts] + [("w", w, (C, 1, k, k))] +
             [(n, t, (C, 1, k, k) if n == "dw" else (C,)) for n, t in others])
    _expect(x.dtype, specs)
    _on_gpu(x, [(n, t) for n, t, _ in specs])


def dwconv_workspace_size(shape):
    n = ctypes.c_size_t(0)
    _check(lib.dwconv_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "dwconv_workspace_size")
    return int(n.value)


def dwconv_fwd(x, w, bias, y=None, stream=None):
    """y = depthwise conv of x with w [C, 1, k, k] plus bias [C]; returns y."""
    _check_dw(x, w, [("x", x), ("y", y)], [("bias", bias)])
    s = dw_shape_of(x, w)
    if y is None:
        y = torch.empty_like(x)
    _check(lib.dwconv_fwd(ctypes.byref(s), _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                          _stream(stream, x.device)), "dwconv_fwd")
    return y


def dwconv_bwd(x, dy, w, dx=None, dw=None, db=None, workspace=None, stream=None):
    """(dx, dw, db) of the depthwise conv in one pass."""
    _check_dw(x, w, [("x", x), ("dy", dy), ("dx", dx)], [("dw", dw), ("db", db)])
    _expect(None, [("workspace", workspace, None)])
    _on_gpu(x, [("workspace", workspace)])
    s = dw_shape_of(x, w)
    dx = torch.empty_like(dy) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    db = torch.empty(w.shape[0], dtype=w.dtype, device=w.device) if db is None else db
    need = dwconv_workspace_size(s)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib.dwconv_bwd(ctypes.byref(s), _ptr(x), _ptr(dy), _ptr(w), _ptr(dx), _ptr(dw),
                          _ptr(db), _ptr(workspace), workspace.numel() * workspace.element_size(),
                          _stream(stream, x.device)), "dwconv_bwd")
    return dx, dw, db
