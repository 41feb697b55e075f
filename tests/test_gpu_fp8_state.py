"""GPU parity of the 8-bit state (E4M3 codes scaled by a power of two)
against the oracle's E4M3-state mode, plus exact invariants of that mode on
the GPU: the codes agree with torch's float32 -> float8_e4m3fn conversion,
doubling the inputs and the scale doubles the results, a continuation split
gives the same bits."""
import numpy as np
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import (FP8_SCALE_LOG2, TOL_FP8, Timer, check_bf16_state, gpu_forward, log,
                      make_core, upload)

pytestmark = pytest.mark.gpu

F8 = torch.float8_e4m3fn


def _parity(wl, c0=0, c1=None, d=None, s=FP8_SCALE_LOG2):
    log(f"fp8 state (scale 2^{s}): {wl.name} B={wl.B} T={wl.T} H={wl.H} S={wl.sqrtN} "
        f"d_v={wl.d_v} W={wl.W} R={wl.R} {wl.dtype} cols=[{c0},{c1 if c1 is not None else wl.d_v})")
    if d is None:
        d = si.generate(wl)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, F8, s)
    assert M.dtype == F8
    c1 = wl.d_v if c1 is None else c1
    ref = oracle.forward(d, wl.sqrtN, wl.W, wl.R, c0=c0, c1=c1, state="fp8", scale_log2=s)
    Mv = core.state_values(M[..., c0:c1])
    check_bf16_state(y[..., c0:c1].double().cpu().numpy(), Mv.double().cpu().numpy(), ref["y"],
                     ref["M"], outer=TOL_FP8)
    return d, core, dd, y, M


SHAPES = [
    # (B, T, H, sqrtN, d_v, W, R, dtype, reuse, scale_log2)
    (1, 64, 1, 16, 32, 4, 4, "f32", 0.0, -4),
    (2, 37, 3, 8, 20, 3, 5, "f32", 0.0, -4),       # ragged column slice, W != R
    (1, 1, 1, 1, 4, 1, 1, "f32", 0.0, -4),         # N = 1, single token
    (2, 300, 2, 16, 72, 16, 16, "f32", 0.3, -5),   # several epochs, key reuse
    (1, 257, 2, 128, 64, 64, 64, "f32", 0.3, -4),  # the 1.4B-style slot count
    (1, 91, 1, 32, 36, 32, 20, "bf16", 0.5, -3),   # bf16 inputs
    (2, 150, 2, 16, 160, 8, 8, "f32", 0.2, 0),     # unscaled codes (subnormal M_0), 2 slices
    # 256 (sequence, head, 64-column) units fill the GPU: epochs of 256
    # tokens (a float32 state would take 512) in one launch
    (4, 1200, 4, 64, 1024, 8, 8, "f32", 0.2, -4),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:7] + (s[9],)) for s in SHAPES])
def test_fp8_state_shapes(shape):
    B, T, H, S, D, W, R, dt, reuse, sc = shape
    wl = si.Workload("fp8 state", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt,
                     reuse=reuse, seed=800 + T)
    _parity(wl, s=sc)


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_fp8_state_full_workload(cfg):
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


def _codes(x: torch.Tensor, s: int) -> torch.Tensor:
    """torch's E4M3 codes of x * 2^-s, as bytes."""
    return (x.float() * 2.0 ** -s).to(F8).view(torch.uint8)


def _e4m3_grid():
    """Every finite E4M3 value, every point halfway between neighbours, and
    random magnitudes over all binades up to 448, with both signs (float32)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(F8).float().numpy()
    vals = np.unique(codes[np.isfinite(codes) & (codes >= 0)]).astype(np.float64)
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(3)
    rnd = np.exp2(rng.uniform(-12, np.log2(448.0), 4096))
    g = np.concatenate([vals, mids, rnd]).astype(np.float32)
    return np.concatenate([g, -g])


def test_fp8_state_init_and_unselected_rows():
    """Rows never written hold the codes of M_0 * 2^-s, bit for bit as
    torch converts them (nearest, ties to even), for M_0 covering every
    E4M3 value, every halfway point and the subnormals."""
    wl, d = _small(51)
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    s = FP8_SCALE_LOG2
    grid = _e4m3_grid() * np.float32(2.0 ** s)
    d["M0"] = np.resize(grid, d["M0"].size).reshape(d["M0"].shape).astype(np.float32)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, F8, s)
    Iw = core.select(dd["kp"], dd["qp"])[0].cpu().numpy()
    want = _codes(dd["M0"], s)
    Mb = M.view(torch.uint8)
    for b in range(wl.B):
        for h in range(wl.H):
            never = np.setdiff1d(np.arange(wl.N), np.unique(Iw[b, :, h]))
            assert never.size > 0
            idx = torch.from_numpy(never).cuda()
            assert torch.equal(Mb[b, h, idx], want[h, idx])


def test_fp8_state_overwrite_gate():
    """alpha = beta = 1 and W = 1: a written row becomes the codes of v_t * 2^-s."""
    wl, d = _small(52, W=1, R=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    s = -3
    core, dd, y, M = gpu_forward(d, 1, 1, sdm.AUTO, F8, s)
    Iw = core.select(dd["kp"], dd["qp"])[0].cpu().numpy()
    vb = _codes(dd["v"], s)
    Mb = M.view(torch.uint8)
    for b in range(wl.B):
        for h in range(wl.H):
            last = {int(Iw[b, t, h, 0]): t for t in range(wl.T)}
            for sl, t in last.items():
                assert torch.equal(Mb[b, h, sl], vb[b, t, h])


def test_fp8_state_saturates():
    """A value beyond 448 * 2^s is held as +-448 * 2^s (the reading
    saturates; the format has no infinities)."""
    wl, d = _small(53, W=1, R=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    d["v"] = (d["v"] * 100.0).astype(np.float32)  # |v| up to a few hundred
    s = -4  # largest magnitude 28
    core, dd, y, M = gpu_forward(d, 1, 1, sdm.AUTO, F8, s)
    ref = oracle.forward(d, wl.sqrtN, 1, 1, state="fp8", scale_log2=s)
    Mv = core.state_values(M).double().cpu().numpy()
    np.testing.assert_array_equal(Mv, ref["M"])
    assert np.abs(Mv).max() == 448.0 * 2.0 ** s
    assert torch.isfinite(y).all()


def test_fp8_state_scaling_by_two_is_exact():
    """2 M_0 and 2 v with the scale 2^(s+1) give the same codes and 2 y."""
    wl, d = _small(54, T=120)
    _, _, y1, M1 = gpu_forward(d, wl.W, wl.R, sdm.AUTO, F8, -4)
    d2 = dict(d)
    d2["M0"] = d["M0"] * 2
    d2["v"] = d["v"] * 2
    _, _, y2, M2 = gpu_forward(d2, wl.W, wl.R, sdm.AUTO, F8, -3)
    assert torch.equal(y2, 2 * y1) and torch.equal(M2.view(torch.uint8), M1.view(torch.uint8))


def test_fp8_state_deterministic_staged_and_continued():
    """Bitwise run-to-run determinism; sdm_forward equals prepare + apply bit
    for bit; a continuation split gives the same state and y bit for bit."""
    wl = si.Workload("fp8 pipe", B=4, T=1189, H=4, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.2, seed=55)
    d = si.generate(wl)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, sdm.AUTO, F8)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    y2, M2 = core.forward(*args)
    y3, M3 = core.forward(*args, staged=True)
    k = 500
    first = [a[:, :k].contiguous() for a in args]
    rest = [a[:, k:].contiguous() for a in args]
    y4, M4 = core.forward(*first)
    y5, M5 = core.forward(*rest, M=M4, cont=True)
    torch.cuda.synchronize()
    u8 = lambda x: x.view(torch.uint8)
    assert torch.equal(y, y2) and torch.equal(u8(M), u8(M2))
    assert torch.equal(y, y3) and torch.equal(u8(M), u8(M3))
    assert torch.equal(u8(M5), u8(M))
    assert torch.equal(torch.cat([y4, y5], 1), y)


def test_fp8_state_rejects_serial_schedule_and_backward():
    wl, d = _small(56)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R, F8)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    with pytest.raises(sdm.SDMError) as e:
        core.forward(*args, variant=sdm.SERIAL)
    assert e.value.status == 2
    with pytest.raises(sdm.SDMError):  # a bfloat16 M for an E4M3-state handle
        core.forward(*args, M=torch.zeros((wl.B, wl.H, wl.N, wl.d_v), device="cuda",
                                          dtype=torch.bfloat16))
    with pytest.raises(sdm.SDMError) as e:
        core.backward(*args, torch.zeros_like(dd["v"]))
    assert e.value.status == 2
