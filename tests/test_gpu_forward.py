"""GPU parity of sdm_forward (select + write + read) against the float64 oracle,
plus exact invariants of the recurrence checked on the GPU alone."""
import numpy as np
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import (TOL, TOL_LONG, Timer, assert_close, check_selection, gpu_forward, log,
                      make_core, to_dev, upload)

pytestmark = pytest.mark.gpu


def _parity(wl, T=None, c0=0, c1=None, tol=TOL, variant=sdm.AUTO, d=None):
    log(f"forward: {wl.name} B={wl.B} T={T or wl.T} H={wl.H} S={wl.sqrtN} d_v={wl.d_v} "
        f"W={wl.W} R={wl.R} {wl.dtype} cols=[{c0},{c1 if c1 is not None else wl.d_v})")
    if d is None:
        d = si.generate(wl, T=T)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, variant)
    c1 = wl.d_v if c1 is None else c1
    ref = oracle.forward(d, wl.sqrtN, wl.W, wl.R, c0=c0, c1=c1)
    Iw, kw, Ir, qw = [o.cpu().numpy() for o in core.select(dd["kp"], dd["qp"])]
    check_selection(Iw, kw, ref["Iw"], ref["kw"], "write set")
    check_selection(Ir, qw, ref["Ir"], ref["qw"], "read set")
    ey = assert_close(y[..., c0:c1].cpu().numpy(), ref["y"], tol, "y")
    eM = assert_close(M[..., c0:c1].cpu().numpy(), ref["M"], tol, "M")
    log(f"  max rel err y {ey:.2e}  M {eM:.2e}")
    return d, dd, y, M


VARIANTS = [sdm.SERIAL, sdm.TIMEPAR]
VNAMES = ["serial", "timepar"]


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_forward_tiny_workload(variant):
    _parity(si.WORKLOADS[0], variant=variant)


SHAPES = [
    # (B, T, H, sqrtN, d_v, W, R, dtype, reuse)
    (2, 37, 3, 8, 20, 3, 5, "f32", 0.0),      # ragged column slice, W != R
    (1, 13, 1, 4, 30, 4, 2, "f32", 0.0),      # d_v % 4 != 0: one-column-per-lane path
    (1, 1, 1, 1, 4, 1, 1, "f32", 0.0),        # N = 1, single token
    (2, 200, 2, 16, 48, 16, 16, "f32", 0.0),  # W = R = sqrtN
    (1, 257, 2, 128, 64, 64, 64, "f32", 0.3),  # the 1.4B-style slot count, key reuse
    (1, 91, 1, 32, 36, 32, 20, "bf16", 0.5),   # bf16 inputs
    (3, 50, 1, 9, 8, 9, 9, "f32", 0.0),       # every token writes 9 of 81 slots
    (1, 300, 1, 1024, 8, 64, 64, "f32", 0.2),  # the largest sqrtN (2^20 slots), W = R = 64
    (2, 600, 1, 512, 16, 64, 32, "bf16", 0.2),  # sqrtN = 512 with bf16 inputs, W != R
]


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:7]) for s in SHAPES])
def test_forward_shapes(shape, variant):
    B, T, H, S, D, W, R, dt, reuse = shape
    if variant == sdm.TIMEPAR and D % 4:
        pytest.skip("the time-parallel schedule needs d_v % 4 == 0 (rejected, tested below)")
    wl = si.Workload("shape", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt, reuse=reuse,
                     seed=500 + T)
    _parity(wl, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_forward_same_keys_every_token(variant):
    """Every token writes the same slots and reads them back: each row is
    rewritten at every step, so every reference goes through the forwarding
    path (previous token for writes, same token for reads)."""
    wl = si.Workload("same keys", B=2, T=64, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.0, seed=9)
    d = si.generate(wl)
    d["kp"][:] = d["kp"][:, :1]
    d["qp"][:] = d["kp"]
    _parity(wl, d=d, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_forward_clustered_keys(variant):
    """Keys drawn from a few prototypes: slots recur at distances 1..8."""
    wl = si.Workload("clustered", B=1, T=300, H=2, sqrtN=32, d_v=64, W=32, R=32, dtype="f32",
                     reuse=0.0, seed=10)
    d = si.generate(wl)
    rng = np.random.default_rng(3)
    proto = d["kp"][0, :5].copy()
    pick = rng.integers(0, 5, size=wl.T)
    d["kp"][0] = proto[pick] + 0.05 * rng.standard_normal(d["kp"][0].shape).astype(np.float32)
    d["qp"][0] = proto[rng.integers(0, 5, size=wl.T)]
    _parity(wl, d=d, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_forward_full_workload(cfg, variant):
    """The full workload on the GPU; the oracle computes every token of every
    chain for a window of 16 columns (columns never interact)."""
    wl = si.WORKLOADS[cfg]
    tol = TOL_LONG if cfg == 4 else TOL
    c0 = {1: 496, 2: 504, 3: 0, 4: 1024}[cfg]
    with Timer("generate"):
        d = si.generate(wl)
    with Timer("gpu + oracle"):
        _parity(wl, d=d, c0=c0, c1=c0 + 16, tol=tol, variant=variant)


# ---------------------------------------------------------------- invariants

def _small(seed, **kw):
    p = dict(B=2, T=40, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32", reuse=0.0, seed=seed)
    p.update(kw)
    wl = si.Workload("inv", **p)
    return wl, si.generate(wl)


def test_unselected_rows_bit_unchanged():
    wl, d = _small(21)
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    core, dd, y, M = gpu_forward(d, wl.W, wl.R)
    Iw = core.select(dd["kp"], dd["qp"])[0].cpu().numpy()
    M = M.cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            never = np.setdiff1d(np.arange(wl.N), np.unique(Iw[b, :, h]))
            assert never.size > wl.N // 2
            np.testing.assert_array_equal(M[b, h, never], d["M0"][h, never])


def test_overwrite_gate_sets_row_to_v():
    """alpha = beta = 1, W = 1 (k = 1): a written row equals v_t bit for bit."""
    wl, d = _small(22, W=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    core, dd, y, M = gpu_forward(d, 1, wl.R)
    Iw = core.select(dd["kp"], dd["qp"])[0].cpu().numpy()
    M = M.cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            last = {int(Iw[b, t, h, 0]): t for t in range(wl.T)}
            for s, t in last.items():
                np.testing.assert_array_equal(M[b, h, s], d["v"][b, t, h])


def _row_equal(variant, got, row):
    """The token-serial read sums the stored rows, so a read of one row with
    weight 1 returns it bit for bit.  The time-parallel read of a float32
    state sums the slot's epoch-start row and the v rows of its earlier
    in-epoch writes with composed weights (A and C_k of the composed affine
    map): the same value up to float32 rounding of that regrouping."""
    if variant == sdm.SERIAL:
        np.testing.assert_array_equal(got, row)
    else:
        np.testing.assert_allclose(got, row, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_one_hot_read_returns_row(variant):
    """R = 1 (q = 1): y of the last token is the final row of its read slot."""
    wl, d = _small(23, R=1)
    core, dd, y, M = gpu_forward(d, wl.W, 1, variant)
    Ir = core.select(dd["kp"], dd["qp"])[2].cpu().numpy()
    y, M = y.cpu().numpy(), M.cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            _row_equal(variant, y[b, -1, h], M[b, h, Ir[b, -1, h, 0]])


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_dominant_read_weight(variant):
    """A score gap above 800 leaves weight 1 on one slot and exactly 0 elsewhere."""
    wl, d = _small(24, R=4)
    S = wl.sqrtN
    d["qp"][:] = 0.0
    d["qp"][..., 0] = 900.0
    d["qp"][..., S + 1:] = -900.0
    core, dd, y, M = gpu_forward(d, wl.W, 4, variant)
    _, _, Ir, qw = [o.cpu().numpy() for o in core.select(dd["kp"], dd["qp"])]
    assert (Ir[..., 0] == 0).all() and (qw[..., 0] == 1).all() and (qw[..., 1:] == 0).all()
    _row_equal(variant, y[:, -1].cpu().numpy(), M[:, :, 0].cpu().numpy())


def test_scaling_by_two_is_exact():
    wl, d = _small(25, sqrtN=32, d_v=64, W=32, R=32, T=120)
    _, _, y1, M1 = gpu_forward(d, wl.W, wl.R)
    d2 = dict(d, M0=d["M0"] * 2, v=d["v"] * 2)
    _, _, y2, M2 = gpu_forward(d2, wl.W, wl.R)
    assert torch.equal(y2, 2 * y1) and torch.equal(M2, 2 * M1)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_runs_are_bitwise_deterministic(variant):
    wl, d = _small(26, sqrtN=64, d_v=128, W=64, R=64, T=200, B=1)
    core, dd, y1, M1 = gpu_forward(d, wl.W, wl.R, variant)
    y2, M2 = core.forward(dd["kp"], dd["qp"], dd["v"], dd["alpha"], dd["beta"], variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(M1, M2)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_continue_flag_splits_a_sequence(variant):
    """Two calls (the second continuing from the first's state) give the same
    outputs as one call over the whole sequence."""
    wl, d = _small(27, sqrtN=32, d_v=64, W=16, R=16, T=90)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, variant)
    k = 37
    part = {n: dd[n][:, :k].contiguous() for n in ("kp", "qp", "v", "alpha", "beta")}
    rest = {n: dd[n][:, k:].contiguous() for n in ("kp", "qp", "v", "alpha", "beta")}
    y1, M1 = core.forward(part["kp"], part["qp"], part["v"], part["alpha"], part["beta"],
                          variant=variant)
    y2, M2 = core.forward(rest["kp"], rest["qp"], rest["v"], rest["alpha"], rest["beta"],
                          M=M1, cont=True, variant=variant)
    torch.cuda.synchronize()
    _same_run(torch.cat([y1, y2], 1), M2, y, M, variant)


def _same_run(y1, M1, y, M, variant):
    """M is bit-exact under any split of the tokens.  So is y with the
    token-serial schedule; the time-parallel read groups its terms by epoch,
    so where a split moves the epoch boundaries y agrees to float32 rounding."""
    assert torch.equal(M1, M)
    if variant == sdm.SERIAL:
        assert torch.equal(y1, y)
    else:
        assert torch.allclose(y1, y, rtol=1e-5, atol=1e-6)


def test_forward_rejects_bad_tensors():
    wl, d = _small(28)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    with pytest.raises(sdm.SDMError):
        core.forward(dd["kp"], dd["qp"], dd["v"].to(torch.bfloat16), dd["alpha"], dd["beta"])
    with pytest.raises(sdm.SDMError):
        core.forward(dd["kp"][:, :, :1], dd["qp"], dd["v"], dd["alpha"], dd["beta"])
    with pytest.raises(sdm.SDMError) as e:
        core.forward(dd["kp"], dd["qp"], dd["v"], dd["alpha"], dd["beta"], variant=7)
    assert e.value.status == 1
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    B, T = wl.B, wl.T
    y_ok = torch.empty((B, T, wl.H, wl.d_v), device="cuda")
    M_ok = torch.empty((B, wl.H, wl.N, wl.d_v), device="cuda")
    need = core.workspace_size(B, T)
    # caller-supplied outputs and workspace are checked on the host: wrong
    # device, dtype, shape or size raise before anything is enqueued
    bad_out = [dict(y=y_ok.cpu()), dict(y=y_ok[:, :-1]), dict(M=M_ok.cpu()), dict(M=M_ok[:1]),
               dict(M=M_ok.to(torch.bfloat16)),
               dict(workspace=torch.empty(need, dtype=torch.uint8)),
               dict(workspace=torch.empty(need // 4 + 1, dtype=torch.float32, device="cuda")),
               dict(workspace=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))]
    for kw in bad_out:
        kw = {**dict(y=y_ok, M=M_ok), **kw}
        with pytest.raises(sdm.SDMError):
            core.forward(*args, **kw)
    with pytest.raises(sdm.SDMError):
        core.forward_noalloc(*args, y=y_ok.cpu(), M=M_ok)
    Iw, kw_, Ir, qw = core.select(dd["kp"], dd["qp"])
    for bad in ((Iw.cpu(), kw_, Ir, qw), (Iw, kw_[:, :1], Ir, qw), (Iw, kw_, Ir.float(), qw),
                (Iw, kw_, Ir, qw.transpose(0, 1))):
        with pytest.raises(sdm.SDMError):
            core.select(dd["kp"], dd["qp"], out=bad)
    with pytest.raises(sdm.SDMError):
        core.write_histogram(dd["kp"], torch.zeros((wl.H, wl.N), dtype=torch.int32))
    wl2, d2 = _small(29, d_v=30)
    dd2 = upload(d2)
    core2 = make_core(dd2, wl2.W, wl2.R)
    with pytest.raises(sdm.SDMError) as e:
        core2.forward(dd2["kp"], dd2["qp"], dd2["v"], dd2["alpha"], dd2["beta"],
                      variant=sdm.TIMEPAR)
    assert e.value.status == 2


@pytest.mark.parametrize("shape", [
    (2, 300, 2, 32, 64, 32, 32, 0.0), (1, 700, 1, 64, 96, 64, 64, 0.4),
    (4, 129, 2, 16, 32, 16, 8, 0.0),
    # 256 units of 128-byte slices: four waves per unit, two references per row group
    (2, 300, 4, 64, 1024, 64, 64, 0.2),
    # 1024 such units: one wave per unit
    (4, 160, 8, 64, 1024, 64, 48, 0.0),
    # ragged last slice (28 of 32 columns) in each kernel form
    (2, 100, 4, 32, 1020, 32, 32, 0.0),
    (4, 64, 8, 32, 1020, 24, 32, 0.0),
    # odd W != R over four waves: 10 write and 8 read positions per wave
    (2, 150, 4, 64, 1024, 37, 29, 0.3),
])
def test_schedules_agree_bitwise_on_state(shape):
    """Both schedules apply the same float32 operations to every row in the
    same order, so the final state agrees bit for bit.  y agrees to float32
    rounding: the time-parallel read sums epoch-start rows and v rows with
    composed weights instead of replaying each write."""
    B, T, H, S, D, W, R, reuse = shape
    wl = si.Workload("agree", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype="f32",
                     reuse=reuse, seed=40 + T)
    d = si.generate(wl)
    _, _, y1, M1 = gpu_forward(d, W, R, sdm.SERIAL)
    _, _, y2, M2 = gpu_forward(d, W, R, sdm.TIMEPAR)
    assert torch.equal(M1, M2)
    assert torch.allclose(y1, y2, rtol=1e-5, atol=1e-6)


def test_schedules_agree_bitwise_with_bf16_inputs():
    """bfloat16 k', q', v (widened exactly) at a shape whose 256 units of
    128-byte slices take the four-wave token-serial kernel: the final state
    agrees bit for bit with the time-parallel schedule."""
    wl = si.Workload("agree bf16", B=2, T=200, H=4, sqrtN=32, d_v=1024, W=32, R=32,
                     dtype="bf16", reuse=0.1, seed=48)
    d = si.generate(wl)
    _, _, y1, M1 = gpu_forward(d, wl.W, wl.R, sdm.SERIAL)
    _, _, y2, M2 = gpu_forward(d, wl.W, wl.R, sdm.TIMEPAR)
    assert torch.equal(M1, M2)
    assert torch.allclose(y1, y2, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_decode_token_by_token(variant):
    """Decoding one token per call (continuing from the previous state) gives
    the same y and M as one call over the whole sequence."""
    wl, d = _small(30, sqrtN=16, d_v=32, W=8, R=8, T=12, B=2, H=2)
    core, dd, y, M = gpu_forward(d, wl.W, wl.R, variant)
    M1 = torch.empty_like(M)
    ys = []
    for t in range(wl.T):
        step = {n: dd[n][:, t:t + 1].contiguous() for n in ("kp", "qp", "v", "alpha", "beta")}
        yt, _ = core.forward(step["kp"], step["qp"], step["v"], step["alpha"], step["beta"],
                             M=M1, cont=t > 0, variant=variant)
        ys.append(yt)
    torch.cuda.synchronize()
    _same_run(torch.cat(ys, 1), M1, y, M, variant)


@pytest.mark.parametrize("shape", [(4, 1189, 4, 16, 32, 8, 8, "f32"),
                                   (2, 1100, 8, 32, 64, 32, 32, "bf16")],
                         ids=["38-epochs", "35-epochs-bf16"])
def test_forward_matches_staged_many_epochs(shape):
    """Many epochs of the time-parallel schedule (the last one partial): the
    forward matches the oracle and gives, bit for bit, what sdm_prepare +
    sdm_apply give: from M_0, continuing from a state, and issued on a
    non-default torch stream whose results are consumed on that stream."""
    B, T, H, S, D, W, R, dt = shape
    wl = si.Workload("epochs", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt, reuse=0.2,
                     seed=60 + T)
    d, dd, y, M = _parity(wl, variant=sdm.TIMEPAR)
    core = make_core(dd, W, R)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    y2, M2 = core.forward(*args, variant=sdm.TIMEPAR, staged=True)
    y3, M3 = core.forward(*args, variant=sdm.TIMEPAR, M=M.clone(), cont=True)
    y4, M4 = core.forward(*args, variant=sdm.TIMEPAR, M=M.clone(), cont=True, staged=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(M, M2)
    assert torch.equal(y3, y4) and torch.equal(M3, M4)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y5, M5 = core.forward(*args, variant=sdm.TIMEPAR)
        s5 = (y5.sum(), M5.sum())  # consumed on the same stream right away
    side.synchronize()
    assert torch.equal(y5, y) and torch.equal(M5, M)
    assert s5[0].item() == y.sum().item() and s5[1].item() == M.sum().item()
