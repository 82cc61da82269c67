"""The Python binding checks tensor metadata before calling the library: the
library sees only pointers and sizes, so a tensor of another shape, dtype or
device would be read out of bounds or as host memory.  CPU only: every call
here is refused before any library call."""
import pytest
import torch

import wtconv_inputs as wi
from aware_conv_amd import _lib as L

PARAMS = ("w_base", "b_base", "s_base", "w_wav", "s_wav")


@pytest.fixture()
def d():
    return wi.make_inputs(2, 3, 16, 16, 2, 5, "f32", seed=0)


def params(d, **over):
    p = {n: d[n] for n in PARAMS}
    p.update(over)
    return [p[n] for n in PARAMS]


def test_host_tensors_are_refused(d):
    with pytest.raises(ValueError, match="GPU"):
        L.wtconv_fwd(d["x"], *params(d))
    with pytest.raises(ValueError, match="GPU"):
        L.wtconv_bwd(d["x"], d["dy"], *params(d))
    with pytest.raises(ValueError, match="GPU"):
        L.dwconv_fwd(d["x"], d["w_base"], d["b_base"])


@pytest.mark.parametrize("name,bad", [
    ("w_base", torch.zeros(2, 1, 5, 5)),          # fewer channels
    ("b_base", torch.zeros(4)),
    ("s_base", torch.zeros(3, 1)),
    ("w_wav", torch.zeros(2, 3, 4, 3, 3)),        # another kernel size
    ("s_wav", torch.zeros(1, 3, 4)),              # fewer levels
])
def test_parameter_shapes_must_match_the_layer(d, name, bad):
    with pytest.raises(ValueError, match="shape"):
        L.wtconv_fwd(d["x"], *params(d, **{name: bad}))


def test_activation_and_output_shapes(d):
    with pytest.raises(ValueError, match="4-D"):
        L.wtconv_fwd(d["x"][0], *params(d))
    with pytest.raises(ValueError, match="dy has shape"):
        L.wtconv_bwd(d["x"], d["dy"][:1], *params(d))
    with pytest.raises(ValueError, match="y has shape"):
        L.wtconv_fwd(d["x"], *params(d), y=torch.empty(2, 3, 16, 8))
    with pytest.raises(ValueError, match="w_wav must be"):
        L.wtconv_fwd(d["x"], *params(d, w_wav=torch.zeros(2, 3, 5, 5)))


def test_dtype_and_layout(d):
    with pytest.raises(TypeError, match="dtype"):
        L.wtconv_fwd(d["x"], *params(d, s_base=d["s_base"].half()))
    with pytest.raises(ValueError, match="contiguous"):
        L.wtconv_fwd(d["x"].transpose(2, 3), *params(d))


def test_gradient_buffers(d):
    g = {n: torch.empty_like(d[p]) for n, p in zip(L.GRAD_NAMES, PARAMS)}
    del g["ds_wav"]
    with pytest.raises(KeyError, match="ds_wav"):
        L.wtconv_bwd_weight(d["x"], d["dy"], *params(d), grads=g)
    g["ds_wav"] = torch.empty(2, 3, 3)
    with pytest.raises(ValueError, match=r"grads\[ds_wav\] has shape"):
        L.wtconv_bwd(d["x"], d["dy"], *params(d), grads=g)


def test_depthwise_baseline_checks(d):
    with pytest.raises(ValueError, match="bias has shape"):
        L.dwconv_fwd(d["x"], d["w_base"], torch.zeros(4))
    with pytest.raises(ValueError, match="w must be"):
        L.dwconv_fwd(d["x"], d["w_base"][:, 0], d["b_base"])


@pytest.mark.gpu
def test_gpu_call_with_a_host_tensor_is_refused(d):
    g = {n: v.cuda() for n, v in d.items()}
    p = params(g, s_base=d["s_base"])  # left on the host
    with pytest.raises(ValueError, match="s_base is on cpu"):
        L.wtconv_fwd(g["x"], *p)
    with pytest.raises(ValueError, match="workspace is on cpu"):
        L.wtconv_bwd(g["x"], g["dy"], *params(g), workspace=torch.empty(1 << 20, dtype=torch.uint8))
