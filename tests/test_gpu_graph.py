"""The C-ABI calls captured into a HIP graph (as a training loop that
captures its step runs them) give, on every replay, the bits of the eager
calls.  The calls allocate nothing and record no memset, so capture needs
nothing beyond preallocated outputs and workspace.  Replays are separated
by other eager work and synchronisation, and each replay is checked."""
import pytest
import torch

import wtconv_inputs as wi

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,B", [("stage1", 8), ("stage3", 8), ("highres", 1)])
def test_graph_replays_match_eager(name, B):
    from aware_conv_amd import _lib as L
    wl = wi.WORKLOADS[name]
    print("\ncase graph %s B=%d" % (name, B), flush=True)
    d = {k: v.cuda() for k, v in wi.workload_inputs(wl, batch=B).items()}
    p = [d[n] for n in ("w_base", "b_base", "s_base", "w_wav", "s_wav")]
    s = L.shape_of(d["x"], d["w_wav"])
    ws = torch.empty(max(16, L.wtconv_workspace_size(s)), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    dx = torch.empty_like(d["x"])
    g = {n: torch.empty_like(t) for n, t in zip(L.GRAD_NAMES, p)}

    def step():
        st = torch.cuda.current_stream()
        L.wtconv_fwd(d["x"], *p, y=y, workspace=ws, stream=st)
        L.wtconv_bwd(d["x"], d["dy"], *p, dx=dx, grads=g, workspace=ws, stream=st)

    step()
    torch.cuda.synchronize()
    ref = [y.clone(), dx.clone()] + [g[n].clone() for n in L.GRAD_NAMES]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in [y, dx] + list(g.values()):
            t.fill_(float("nan"))
        # unrelated eager work between replays, then a full synchronisation
        junk = torch.randn(1 << 20, device="cuda").cumsum(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [y, dx] + [g[n] for n in L.GRAD_NAMES]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), (name, rep)
        del junk
