"""sdm_forward_noalloc (the forward with the library's static scratch instead
of a workspace) against sdm_forward on the same inputs: the two run the same
kernels, so y and M must agree bit for bit.  Two calls in a row, the second
with a smaller input, so the second runs on scratch the first left behind."""
import pytest
import torch

import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import log, make_core, upload

pytestmark = pytest.mark.gpu

NAMES = ("kp", "qp", "v", "alpha", "beta")


def _pair(core, dd, B, T, variant, state):
    """(y, M) from sdm_forward and from sdm_forward_noalloc on the first B
    sequences and T tokens of dd."""
    args = [dd[n][:B, :T].contiguous() for n in NAMES]
    y1, M1 = core.forward(*args, variant=variant)
    y2 = torch.full_like(y1, float("nan"))
    M2 = torch.full_like(M1, float("nan"))
    core.forward_noalloc(*args, y=y2, M=M2, variant=variant)
    torch.cuda.synchronize()
    return y1, M1, y2, M2


CASES = [  # (B, T, H, sqrtN, d_v, W, R, dtype, variant, state)
    (3, 300, 2, 32, 64, 32, 32, "f32", sdm.TIMEPAR, torch.float32),
    (2, 130, 2, 16, 48, 8, 12, "bf16", sdm.SERIAL, torch.float32),
    (2, 200, 3, 16, 64, 16, 16, "f32", sdm.AUTO, torch.bfloat16),
    (8, 256, 4, 128, 512, 64, 64, "f32", sdm.TIMEPAR, torch.float32),  # 1.4B-style layer shape
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:8]) for c in CASES])
def test_noalloc_equals_forward_twice(case):
    B, T, H, S, D, W, R, dt, variant, state = case
    wl = si.Workload("noalloc", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt, reuse=0.2,
                     seed=900 + T)
    dd = upload(si.generate(wl))
    core = make_core(dd, W, R, state)
    for Bc, Tc in ((B, T), (max(1, B - 1), T // 3 + 1)):  # second call: smaller
        log(f"noalloc: B={Bc} T={Tc} H={H} S={S} d_v={D} W={W} R={R} {dt} variant={variant} "
            f"state={state}")
        y1, M1, y2, M2 = _pair(core, dd, Bc, Tc, variant, state)
        assert torch.equal(y1, y2) and torch.equal(M1, M2)


def test_noalloc_decode_steps_and_graph():
    """One-token steps continuing the state, eager and from a captured graph
    (the use the entry point is for), equal to sdm_forward's steps."""
    wl = si.Workload("noalloc decode", B=4, T=12, H=2, sqrtN=32, d_v=64, W=16, R=16, dtype="f32",
                     reuse=0.3, seed=77)
    dd = upload(si.generate(wl))
    core = make_core(dd, wl.W, wl.R)
    steps = [[dd[n][:, t:t + 1].contiguous() for n in NAMES] for t in range(wl.T)]
    M_e = torch.empty((wl.B, wl.H, wl.N, wl.d_v), device="cuda")
    M_n = torch.empty_like(M_e)
    y_n = torch.empty((wl.B, 1, wl.H, wl.d_v), device="cuda")
    ys = []
    for t in range(wl.T):
        y, _ = core.forward(*steps[t], M=M_e, cont=t > 0)
        core.forward_noalloc(*steps[t], y=y_n, M=M_n, cont=t > 0)
        torch.cuda.synchronize()
        assert torch.equal(y, y_n), t
        ys.append(y.clone())
    assert torch.equal(M_e, M_n)
    # replay a captured continuation step: token 0 eagerly, then tokens 1.. by replays
    static = [x.clone() for x in steps[1]]
    core.forward_noalloc(*steps[0], y=y_n, M=M_n)
    torch.cuda.synchronize()
    keep = M_n.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        core.forward_noalloc(*static, y=y_n, M=M_n, cont=True)
    M_n.copy_(keep)
    for t in range(1, wl.T):
        for dst, src in zip(static, steps[t]):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_n, ys[t]), t
    assert torch.equal(M_n, M_e)


def test_noalloc_rejects_oversize():
    wl = si.Workload("noalloc big", B=1, T=8, H=1, sqrtN=16, d_v=32, W=4, R=4, dtype="f32",
                     reuse=0.0, seed=1)
    dd = upload(si.generate(wl))
    core = make_core(dd, 4, 4)
    n = core.workspace_size(64, 1 << 14)
    assert n > sdm.NOALLOC_MAX_BYTES
    big = [torch.zeros((64, 1 << 14) + tuple(dd[k].shape[2:]), dtype=dd[k].dtype, device="cuda")
           for k in NAMES]
    y = torch.empty((64, 1 << 14, 1, 32), device="cuda")
    M = torch.empty((64, 1, 256, 32), device="cuda")
    with pytest.raises(sdm.SDMError) as e:
        core.forward_noalloc(*big, y=y, M=M)
    assert e.value.status == 2
