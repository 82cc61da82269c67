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
LIB_PATH = os.path.join(_HERE, "libwtconv.so")

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
            "wtconv_bwd_weight", "wtconv_bwd", "wtconv_strerror",
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


def wtconv_bwd_weight(x, dy, w_base, b_base, s_base, w_wav, s_wav, grads=None,
                      workspace=None, stream=None):
    """Parameter gradients; returns a dict keyed by GRAD_NAMES."""
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


# ---------------------------------------------------------------------------
# Plain depthwise conv baseline (include/dwconv.h)
# ---------------------------------------------------------------------------

def dw_shape_of(x, w):
    B, C, H, W = x.shape
    return DwShape(int(B), int(C), int(H), int(W), int(w.shape[-1]), _dtype_code(x.dtype))


def dwconv_workspace_size(shape):
    n = ctypes.c_size_t(0)
    _check(lib.dwconv_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "dwconv_workspace_size")
    return int(n.value)


def dwconv_fwd(x, w, bias, y=None, stream=None):
    """y = depthwise conv of x with w [C, 1, k, k] plus bias [C]; returns y."""
    s = dw_shape_of(x, w)
    if y is None:
        y = torch.empty_like(x)
    _check(lib.dwconv_fwd(ctypes.byref(s), _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                          _stream(stream, x.device)), "dwconv_fwd")
    return y


def dwconv_bwd(x, dy, w, dx=None, dw=None, db=None, workspace=None, stream=None):
    """(dx, dw, db) of the depthwise conv in one pass."""
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
