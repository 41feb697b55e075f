"""GPU parity of the reduced-precision (bfloat16) state against the oracle's
bfloat16-state mode, plus exact invariants of that mode on the GPU."""
import numpy as np
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import Timer, check_bf16_state, gpu_forward, log, make_core, upload

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _parity(wl, c0=0, c1=None, d=None):
    log(f"bf16 state: {wl.name} B={wl.B} T={wl.T} H={wl.H} S={wl.sqrtN} d_v={wl.d_v} "
        f"W={wl.W} R={wl.R} {wl.dtype} cols=[{c0},{c1 if c1 is not None else wl.d_v})")
    if d is None:
        d = si.generate(wl)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, BF)
    assert M.dtype == BF
    c1 = wl.d_v if c1 is None else c1
    ref = oracle.forward(d, wl.sqrtN, wl.W, wl.R, c0=c0, c1=c1, state="bf16")
    check_bf16_state(y[..., c0:c1].double().cpu().numpy(), M[..., c0:c1].double().cpu().numpy(),
                     ref["y"], ref["M"])
    return d, core, dd, y, M


SHAPES = [
    # (B, T, H, sqrtN, d_v, W, R, dtype, reuse)
    (1, 64, 1, 16, 32, 4, 4, "f32", 0.0),
    (2, 37, 3, 8, 20, 3, 5, "f32", 0.0),       # ragged column slice, W != R
    (1, 1, 1, 1, 4, 1, 1, "f32", 0.0),         # N = 1, single token
    (2, 300, 2, 16, 72, 16, 16, "f32", 0.3),   # several epochs, key reuse
    (1, 257, 2, 128, 64, 64, 64, "f32", 0.3),  # the 1.4B-style slot count
    (1, 91, 1, 32, 36, 32, 20, "bf16", 0.5),   # bf16 inputs
    # 256 (sequence, head, 64-column) units fill the GPU: epochs of 256
    # tokens (a float32 state would take 512) in one launch
    (4, 1200, 4, 64, 1024, 8, 8, "f32", 0.2),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:7]) for s in SHAPES])
def test_bf16_state_shapes(shape):
    B, T, H, S, D, W, R, dt, reuse = shape
    wl = si.Workload("bf16 state", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt,
                     reuse=reuse, seed=700 + T)
    _parity(wl)


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_bf16_state_full_workload(cfg):
    """Full-size workload on the GPU; the oracle recomputes a 16-column window."""
    wl = si.WORKLOADS[cfg]
    with Timer("generate"):
        d = si.generate(wl)
    with Timer("gpu + oracle"):
        _parity(wl, d=d, c0=96, c1=112)


def _small(seed, **kw):
    p = dict(B=2, T=40, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32", reuse=0.0, seed=seed)
    p.update(kw)
    wl = si.Workload("inv", **p)
    return wl, si.generate(wl)


def test_bf16_state_init_and_unselected_rows():
    """Rows never written hold M_0 rounded to bfloat16 (nearest-even), bit for
    bit: the rounding agrees with torch's float32 -> bfloat16 conversion."""
    wl, d = _small(41)
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, BF)
    Iw = core.select(dd["kp"], dd["qp"])[0].cpu().numpy()
    M0b = dd["M0"].to(BF)
    for b in range(wl.B):
        for h in range(wl.H):
            never = np.setdiff1d(np.arange(wl.N), np.unique(Iw[b, :, h]))
            assert never.size > 0
            idx = torch.from_numpy(never).cuda()
            assert torch.equal(M[b, h, idx], M0b[h, idx])


def test_bf16_state_overwrite_gate():
    """alpha = beta = 1 and W = 1: a written row becomes bfloat16(v_t)."""
    wl, d = _small(42, W=1, R=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    core, dd, y, M = gpu_forward(d, 1, 1, sdm.AUTO, BF)
    Iw = core.select(dd["kp"], dd["qp"])[0].cpu().numpy()
    vb = dd["v"].to(BF)
    for b in range(wl.B):
        for h in range(wl.H):
            last = {int(Iw[b, t, h, 0]): t for t in range(wl.T)}
            for s, t in last.items():
                assert torch.equal(M[b, h, s], vb[b, t, h])


def test_bf16_state_scaling_by_two_is_exact():
    wl, d = _small(43, T=120)
    _, _, y1, M1 = gpu_forward(d, wl.W, wl.R, sdm.AUTO, BF)
    d2 = dict(d)
    d2["M0"] = d["M0"] * 2
    d2["v"] = d["v"] * 2
    _, _, y2, M2 = gpu_forward(d2, wl.W, wl.R, sdm.AUTO, BF)
    assert torch.equal(y2, 2 * y1) and torch.equal(M2, 2 * M1)


def test_bf16_state_deterministic_staged_and_continued():
    """Bitwise run-to-run determinism; sdm_forward (which runs on one stream
    with a bfloat16 state) equals prepare + apply bit for bit; a continuation
    split gives the same state and the same y bit for bit: every read sees
    the rows as stored, so y does not depend on where an epoch starts."""
    wl = si.Workload("bf16 pipe", B=4, T=1189, H=4, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.2, seed=44)
    d = si.generate(wl)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, BF)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    y2, M2 = core.forward(*args)
    y3, M3 = core.forward(*args, staged=True)
    k = 500
    first = [a[:, :k].contiguous() for a in args]
    rest = [a[:, k:].contiguous() for a in args]
    y4, M4 = core.forward(*first)
    y5, M5 = core.forward(*rest, M=M4, cont=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(M, M2)
    assert torch.equal(y, y3) and torch.equal(M, M3)
    assert torch.equal(M5, M)
    assert torch.equal(torch.cat([y4, y5], 1), y)


def test_bf16_state_rejects_serial_schedule():
    wl, d = _small(45)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R, BF)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    with pytest.raises(sdm.SDMError) as e:
        core.forward(*args, variant=sdm.SERIAL)
    assert e.value.status == 2
    with pytest.raises(sdm.SDMError):  # a float32 M for a bfloat16-state handle
        core.forward(*args, M=torch.zeros((wl.B, wl.H, wl.N, wl.d_v), device="cuda"))
