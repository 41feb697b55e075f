"""The narrow-state apply in one launch (one workgroup per chain and 64-column
slice takes every epoch: v staged in LDS, reads, then writes) against the
per-epoch launches, bit for bit, with SDM_TP_FUSED forcing either form; and the
fused form against the oracle's bfloat16 / E4M3 modes."""
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import (FP8_SCALE_LOG2, TOL_BF16, TOL_FP8, check_bf16_state, gpu_forward, log,
                      make_core, upload)

pytestmark = pytest.mark.gpu

STATES = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}

SHAPES = [
    # (B, T, H, sqrtN, d_v, W, R, dtype, reuse)
    (2, 37, 3, 8, 20, 3, 5, "f32", 0.0),        # one epoch, a ragged 20-column slice
    (2, 300, 2, 16, 72, 16, 16, "f32", 0.3),    # 19 epochs of 16 tokens, 64 + 8 columns
    (1, 257, 2, 128, 64, 64, 64, "f32", 0.3),   # epochs of 256 tokens, the last of one
    (1, 91, 1, 32, 36, 32, 20, "bf16", 0.5),    # bfloat16 inputs, R = 20
    (2, 600, 2, 64, 64, 16, 40, "f32", 0.9),    # heavy key reuse: reads replay 3+ writes
    (1, 64, 1, 64, 128, 16, 64, "f32", 0.0),    # R = sqrtN = 64, one 64-token epoch, 2 slices
]


def _wl(shape, seed):
    B, T, H, S, D, W, R, dt, reuse = shape
    return si.Workload("fused apply", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt,
                       reuse=reuse, seed=seed)


def _forward(monkeypatch, d, wl, state, mode):
    monkeypatch.setenv("SDM_TP_FUSED", mode)
    _, _, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, STATES[state], FP8_SCALE_LOG2)
    return y, M


@pytest.mark.parametrize("state", ["bf16", "fp8"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:7]) for s in SHAPES])
def test_fused_matches_per_epoch(monkeypatch, shape, state):
    wl = _wl(shape, 900 + shape[1])
    log(f"fused vs per-epoch, {state} state: B={wl.B} T={wl.T} H={wl.H} S={wl.sqrtN} "
        f"d_v={wl.d_v} W={wl.W} R={wl.R} {wl.dtype} reuse={wl.reuse}")
    d = si.generate(wl)
    y0, M0 = _forward(monkeypatch, d, wl, state, "0")
    y1, M1 = _forward(monkeypatch, d, wl, state, "1")
    u8 = lambda x: x.view(torch.uint8)
    assert torch.equal(y0, y1), f"y differs at {(y0 != y1).sum().item()} elements"
    assert torch.equal(u8(M0), u8(M1)), f"M differs at {(u8(M0) != u8(M1)).sum().item()} bytes"


@pytest.mark.parametrize("state", ["bf16", "fp8"])
def test_fused_oracle_parity(monkeypatch, state):
    wl = _wl((2, 300, 2, 16, 72, 16, 16, "f32", 0.3), 931)
    d = si.generate(wl)
    monkeypatch.setenv("SDM_TP_FUSED", "1")
    core, _, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, STATES[state], FP8_SCALE_LOG2)
    kw = {"scale_log2": FP8_SCALE_LOG2} if state == "fp8" else {}
    ref = oracle.forward(d, wl.sqrtN, wl.W, wl.R, state=state, **kw)
    Mv = core.state_values(M) if state == "fp8" else M
    check_bf16_state(y.double().cpu().numpy(), Mv.double().cpu().numpy(), ref["y"], ref["M"],
                     outer=TOL_FP8 if state == "fp8" else TOL_BF16)


def test_fused_continuation_split(monkeypatch):
    """Reads of the stored rows do not depend on where a call (or an epoch)
    starts: a forward split into two calls gives the same y and M bits."""
    wl = _wl((2, 300, 2, 16, 72, 16, 16, "f32", 0.3), 932)
    d = si.generate(wl)
    monkeypatch.setenv("SDM_TP_FUSED", "1")
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, torch.bfloat16)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    k = 123
    y1, M1 = core.forward(*[a[:, :k].contiguous() for a in args])
    y2, M2 = core.forward(*[a[:, k:].contiguous() for a in args], M=M1, cont=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], 1), y)
    assert torch.equal(M2.view(torch.uint8), M.view(torch.uint8))


@pytest.mark.parametrize("state", ["bf16", "fp8"])
def test_fused_graph_replays(monkeypatch, state):
    """The one-launch apply captured in a HIP graph replays bit for bit like
    the eager call (eager work and a synchronisation between replays)."""
    wl = _wl((2, 300, 2, 16, 72, 16, 16, "f32", 0.3), 933)
    monkeypatch.setenv("SDM_TP_FUSED", "1")
    dd = upload(si.generate(wl))
    core = make_core(dd, wl.W, wl.R, STATES[state], FP8_SCALE_LOG2)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    y_e, M_e = core.forward(*args)
    ws = torch.empty(core.workspace_size(wl.B, wl.T, sdm.F32, sdm.AUTO), dtype=torch.uint8,
                     device="cuda")
    y_s, M_s = torch.empty_like(y_e), torch.empty_like(M_e)
    core.forward(*args, y=y_s, M=M_s, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        core.forward(*args, y=y_s, M=M_s, workspace=ws)
    u8 = lambda x: x.view(torch.uint8)
    for rep in range(3):
        y_s.fill_(float("nan"))
        u8(M_s).fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_s, y_e) and torch.equal(u8(M_s), u8(M_e)), rep
        _ = (y_e * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("state", ["bf16", "fp8"])
def test_fused_noalloc(monkeypatch, state):
    """sdm_forward_noalloc takes the same one-launch apply: y and M equal
    sdm_forward's bit for bit, twice (the second call smaller)."""
    wl = _wl((2, 300, 2, 16, 72, 16, 16, "f32", 0.3), 934)
    monkeypatch.setenv("SDM_TP_FUSED", "1")
    dd = upload(si.generate(wl))
    core = make_core(dd, wl.W, wl.R, STATES[state], FP8_SCALE_LOG2)
    u8 = lambda x: x.view(torch.uint8)
    for B, T in ((wl.B, wl.T), (1, 101)):
        args = [dd[n][:B, :T].contiguous() for n in ("kp", "qp", "v", "alpha", "beta")]
        y1, M1 = core.forward(*args)
        y2 = torch.full_like(y1, float("nan"))
        M2 = torch.empty_like(M1)
        u8(M2).fill_(0xFF)
        core.forward_noalloc(*args, y=y2, M=M2)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(u8(M1), u8(M2)), (B, T)
