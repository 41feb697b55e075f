"""HIP graph capture of the forward: many epochs of the time-parallel
schedule, a short sequence, and a one-token decode step
replay bit for bit like eager calls.  Replays are separated by eager work
and synchronisations, and every replay is checked."""
import numpy as np
import pytest
import torch

import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import make_core, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(4, 1189, 4, 16, 32, 8, 8), (2, 300, 2, 32, 64, 16, 16)],
                         ids=["many-epochs", "few-epochs"])
@pytest.mark.parametrize("variant", [sdm.TIMEPAR, sdm.SERIAL], ids=["timepar", "serial"])
def test_forward_graph_replays(shape, variant):
    B, T, H, S, D, W, R = shape
    wl = si.Workload("graph", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype="f32",
                     reuse=0.1, seed=90 + T)
    dd = upload(si.generate(wl))
    core = make_core(dd, W, R)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    y_e, M_e = core.forward(*args, variant=variant)
    ws = torch.empty(core.workspace_size(B, T, sdm.F32, variant), dtype=torch.uint8,
                     device="cuda")
    y_s, M_s = torch.empty_like(y_e), torch.empty_like(M_e)
    core.forward(*args, variant=variant, y=y_s, M=M_s, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        core.forward(*args, variant=variant, y=y_s, M=M_s, workspace=ws)
    for rep in range(3):
        y_s.fill_(float("nan"))
        M_s.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_s, y_e) and torch.equal(M_s, M_e), rep
        _ = (y_e * 2).sum().item()  # eager work between replays


def test_decode_step_graph():
    """A captured one-token step (state continued in place) replayed token by
    token, with the token's inputs copied into static buffers before each
    replay, gives the eager decode bit for bit."""
    wl = si.Workload("graph decode", B=2, T=40, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.0, seed=95)
    dd = upload(si.generate(wl))
    core = make_core(dd, wl.W, wl.R)
    names = ("kp", "qp", "v", "alpha", "beta")
    steps = [[dd[n][:, t:t + 1].contiguous() for n in names] for t in range(wl.T)]
    # eager reference: token by token
    M_e = torch.empty((wl.B, wl.H, wl.N, wl.d_v), device="cuda")
    ys_e = []
    for t in range(wl.T):
        y, _ = core.forward(*steps[t], M=M_e, cont=t > 0)
        ys_e.append(y.clone())
    # graph: token 0 eagerly (initialises M), then a captured continuation step
    static = [x.clone() for x in steps[1]]
    M_g = torch.empty_like(M_e)
    y_g = torch.empty_like(ys_e[0])
    ws = torch.empty(core.workspace_size(wl.B, 1), dtype=torch.uint8, device="cuda")
    core.forward(*steps[0], M=M_g, y=y_g, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_g, ys_e[0])
    M_keep = M_g.clone()
    core.forward(*static, M=M_g, y=y_g, workspace=ws, cont=True)  # warm-up outside capture
    M_g.copy_(M_keep)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        core.forward(*static, M=M_g, y=y_g, workspace=ws, cont=True)
    M_g.copy_(M_keep)  # capture does not run the kernels; restore anyway
    for t in range(1, wl.T):
        for dst, src in zip(static, steps[t]):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, ys_e[t]), t
    assert torch.equal(M_g, M_e)
