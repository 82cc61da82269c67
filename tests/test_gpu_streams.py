"""The library keeps no state between calls: two call sequences issued at
the same time on two streams, each with its own workspace and outputs, give
the bits the same sequences give one after the other."""
import pytest
import torch

import wtconv_inputs as wi

pytestmark = pytest.mark.gpu

PARAMS = ("w_base", "b_base", "s_base", "w_wav", "s_wav")


def run(d):
    from aware_conv_amd import _lib as L
    p = [d[n] for n in PARAMS]
    y = L.wtconv_fwd(d["x"], *p)
    dx, g = L.wtconv_bwd(d["x"], d["dy"], *p)
    dxi = L.wtconv_bwd_input(d["dy"], p[0], p[2], p[3], p[4])
    gw = L.wtconv_bwd_weight(d["x"], d["dy"], *p)
    out = {"y": y, "dx": dx, "dx_input": dxi}
    out.update(g)
    out.update({"split_" + n: v for n, v in gw.items()})
    return out


@pytest.mark.parametrize("B,C,H,W,L,k", [
    (4, 16, 56, 56, 2, 5),      # whole planes
    (2, 3, 128, 192, 4, 5),     # tiles and per-plane deep levels
    (1, 2, 768, 768, 6, 3),     # tiles and deep levels through device memory
    (3, 4, 55, 41, 2, 3),       # zero-extended tiled planes in the workspace
    (4, 16, 55, 55, 2, 5),      # corners of whole planes
])
def test_two_streams_match_sequential_calls(B, C, H, W, L, k):
    dev = torch.device("cuda")
    ins = [{n: v.to(dev) for n, v in wi.make_inputs(B, C, H, W, L, k, "f32", seed=s).items()}
           for s in (1, 2)]
    torch.cuda.synchronize()
    ref = [run(d) for d in ins]
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for rep in range(3):
        for i, st in enumerate(streams):
            st.wait_stream(main)
            with torch.cuda.stream(st):
                got[i] = run(ins[i])
        torch.cuda.synchronize()
        for i in range(2):
            for n, v in ref[i].items():
                assert torch.equal(got[i][n], v), (rep, i, n)
