"""GPU parity of the one-token step (T = 1, time-parallel variant: sdm_forward
runs selection, writes and reads in one launch) against the float64 oracle
run over the whole sequence, against the two-launch form (sdm_prepare +
sdm_apply) bit for bit, plus its exact properties."""
import numpy as np
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import (FP8_SCALE_LOG2, TOL, TOL_BF16, TOL_FP8, assert_close, check_bf16_state, log,
                      make_core, upload)

pytestmark = pytest.mark.gpu

NAMES = ("kp", "qp", "v", "alpha", "beta")


def _decode_run(d, dd, W, R, prefill, state=torch.float32, variant=sdm.TIMEPAR):
    """GPU: the first `prefill` tokens in one call (none: start from M_0 on the
    first step), then one call per remaining token continuing the state.
    Slices are copied into fresh allocations: a view of one token can sit off
    the 16-byte alignment the library requires."""
    core = make_core(dd, W, R, state)
    T = dd["v"].shape[1]
    ys = []
    M = None
    if prefill:
        pre = [dd[n][:, :prefill].contiguous().clone() for n in NAMES]
        y0, M = core.forward(*pre, variant=variant)
        ys.append(y0)
    for t in range(prefill, T):
        step = [dd[n][:, t:t + 1].contiguous().clone() for n in NAMES]
        if M is None:
            yt, M = core.forward(*step, variant=variant)
        else:
            yt, _ = core.forward(*step, variant=variant, M=M, cont=True)
        ys.append(yt)
    torch.cuda.synchronize()
    return core, torch.cat(ys, 1), M


SHAPES = [
    # (B, H, sqrtN, d_v, W, R, dtype, state, prefill, steps)
    (3, 2, 8, 20, 3, 5, "f32", "f32", 0, 6),       # ragged slice (d_v < 32 columns), W != R
    (1, 1, 1, 4, 1, 1, "f32", "f32", 0, 3),        # N = 1: every token rewrites and rereads slot 0
    (2, 2, 16, 48, 16, 16, "f32", "f32", 9, 5),    # W = R = sqrtN, after a prefill
    (2, 1, 9, 8, 9, 9, "f32", "f32", 4, 4),        # every token writes 9 of 81 slots
    (1, 2, 64, 96, 64, 1, "f32", "f32", 3, 4),     # W = 64 (8 rows per lane group), R = 1
    (1, 2, 64, 96, 1, 64, "f32", "f32", 3, 4),     # W = 1, R = 64
    (1, 2, 32, 36, 32, 20, "bf16", "f32", 5, 5),   # bf16 inputs
    (2, 2, 32, 64, 32, 32, "f32", "bf16", 6, 5),   # bfloat16 state
    (1, 1, 16, 100, 16, 4, "bf16", "bf16", 2, 4),  # bfloat16 state, ragged 64-column slice
    (2, 1, 64, 128, 64, 64, "f32", "bf16", 3, 3),  # bfloat16 state, W = R = 64 (16 rows per group)
    (2, 2, 32, 64, 32, 32, "f32", "fp8", 6, 5),    # E4M3 state
    (1, 1, 16, 100, 16, 4, "bf16", "fp8", 2, 4),   # E4M3 state, ragged 64-column slice
    (2, 1, 64, 160, 64, 64, "f32", "fp8", 3, 3),   # E4M3 state, W = R = 64, 3 slices
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_decode_matches_oracle(shape):
    B, H, S, D, W, R, dt, st, prefill, steps = shape
    T = prefill + steps
    wl = si.Workload("decode", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt, reuse=0.3,
                     seed=500 + S + D + W + R)
    log(f"decode: B={B} H={H} S={S} d_v={D} W={W} R={R} {dt} state={st} "
        f"prefill={prefill} steps={steps}")
    d = si.generate(wl)
    dd = upload(d)
    state = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[st]
    core, y, M = _decode_run(d, dd, W, R, prefill, state)
    ref = oracle.forward(d, S, W, R, state=st, scale_log2=FP8_SCALE_LOG2)
    if st != "f32":
        check_bf16_state(y.double().cpu().numpy(), core.state_values(M).double().cpu().numpy(),
                         ref["y"], ref["M"], outer=TOL_FP8 if st == "fp8" else TOL_BF16)
        return
    ey = assert_close(y.cpu().numpy(), ref["y"], TOL, "y")
    eM = assert_close(M.float().cpu().numpy(), ref["M"], TOL, "M")
    log(f"  max rel err y {ey:.2e}  M {eM:.2e}")


def test_decode_state_bitwise_equals_serial():
    """The state after one-token steps is bit for bit what the token-serial
    schedule computes (the same a*row + c*v per write); y agrees to float32
    rounding (its terms are summed in another order)."""
    wl = si.Workload("decode", B=3, T=7, H=2, sqrtN=16, d_v=64, W=12, R=9, dtype="f32", reuse=0.4,
                     seed=41)
    d = si.generate(wl)
    dd = upload(d)
    _, y1, M1 = _decode_run(d, dd, wl.W, wl.R, 0, variant=sdm.TIMEPAR)
    _, y2, M2 = _decode_run(d, dd, wl.W, wl.R, 0, variant=sdm.SERIAL)
    assert torch.equal(M1, M2)
    assert torch.allclose(y1, y2, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_reads_its_own_write(state):
    """With W = R = 1, the same key for writing and reading, and beta = 1, the
    written slot becomes v exactly (a = 0, c = 1) and the read returns it:
    y == v bit for bit, so the read saw the same token's write.  v is
    bfloat16, so the bfloat16 state holds it exactly too."""
    wl = si.Workload("decode", B=4, T=3, H=3, sqrtN=8, d_v=72, W=1, R=1, dtype="bf16", reuse=0.0,
                     seed=7)
    d = si.generate(wl)
    d["qp"] = d["kp"].copy()
    d["beta"] = np.ones_like(d["beta"])
    dd = upload(d)
    _, y, M = _decode_run(d, dd, 1, 1, 0, state)
    assert torch.equal(y, dd["v"].float())


def test_decode_leaves_unselected_rows():
    """Rows no write selected keep their bits from the previous state."""
    wl = si.Workload("decode", B=2, T=2, H=2, sqrtN=16, d_v=32, W=4, R=4, dtype="f32", reuse=0.0,
                     seed=9)
    d = si.generate(wl)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    first = [dd[n][:, :1].contiguous().clone() for n in NAMES]
    _, M = core.forward(*first, variant=sdm.TIMEPAR)
    M_before = M.clone()
    step = [dd[n][:, 1:2].contiguous().clone() for n in NAMES]
    core.forward(*step, variant=sdm.TIMEPAR, M=M, cont=True)
    Iw = core.select(step[0], step[1])[0].cpu().numpy()  # [B][1][H][W]
    torch.cuda.synchronize()
    touched = np.zeros((wl.B, wl.H, wl.sqrtN ** 2), dtype=bool)
    for b in range(wl.B):
        for h in range(wl.H):
            touched[b, h, Iw[b, 0, h]] = True
    keep = torch.from_numpy(~touched).cuda()
    assert torch.equal(M[keep], M_before[keep])
    assert not torch.equal(M[~keep], M_before[~keep])


@pytest.mark.parametrize("cfg", [1, 3, 4], ids=["1.4B-style", "8B-style", "long-context"])
def test_decode_full_layer_columns(cfg):
    """A full layer shape (1.4B-style: 8 sequences x 4 heads, 16,384 slots of
    512 columns; 8B-style: 65,536 slots of 1,024; long-context: one sequence,
    262,144 slots of 2,048, bf16 inputs; W = R = 64): 16 prefill tokens, then
    4 one-token steps; y and M of the first 64 columns against the oracle."""
    wl = si.WORKLOADS[cfg]
    T = 20
    log(f"decode full layer: {wl.name} T={T}")
    d = si.generate(wl, T=T)
    dd = upload(d)
    _, y, M = _decode_run(d, dd, wl.W, wl.R, 16)
    ref = oracle.forward(d, wl.sqrtN, wl.W, wl.R, c0=0, c1=64)
    assert_close(y[..., :64].cpu().numpy(), ref["y"], TOL, "y")
    assert_close(M[..., :64].cpu().numpy(), ref["M"], TOL, "M")


FUSED = [
    # (B, H, sqrtN, d_v, W, R, dtype, state, same keys for writing and reading)
    (3, 2, 8, 20, 3, 5, "f32", "f32", False),       # sqrtN <= 64, ragged slice, W != R
    (2, 2, 100, 96, 64, 64, "f32", "f32", False),   # 64 < sqrtN <= 128, W = R = 64
    (1, 3, 150, 40, 17, 33, "bf16", "f32", False),  # 128 < sqrtN <= 256, bf16 inputs
    (1, 1, 300, 36, 64, 64, "f32", "f32", False),   # 256 < sqrtN <= 512
    (2, 2, 64, 64, 64, 64, "f32", "f32", True),     # every read's slot written by the token
    (2, 2, 64, 128, 64, 64, "f32", "bf16", True),   # the same, bfloat16 state
    (2, 1, 64, 160, 64, 64, "f32", "fp8", True),    # the same, E4M3 state
    (1, 2, 32, 100, 32, 20, "bf16", "bf16", False),
    (1, 2, 32, 100, 20, 32, "bf16", "fp8", False),
    (64, 4, 16, 1000, 8, 8, "f32", "f32", False),   # four row waves, several slices each, ragged
    (8, 4, 16, 512, 16, 16, "f32", "f32", False),   # two row waves per workgroup (256 CUs)
    (8, 4, 16, 2048, 16, 16, "f32", "fp8", True),   # four row waves, E4M3
]


@pytest.mark.parametrize("shape", FUSED, ids=[str(s) for s in FUSED])
def test_fused_step_bitwise_equals_two_launches(shape):
    """sdm_forward's one-launch step (selection inside) gives the bits of
    sdm_prepare + sdm_apply (selection kernel, records, write/read kernel):
    from M_0 and continuing a prefilled state."""
    B, H, S, D, W, R, dt, st, same = shape
    wl = si.Workload("decode", B=B, T=4, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt, reuse=0.3,
                     seed=900 + S + D + W)
    log(f"fused step: B={B} H={H} S={S} d_v={D} W={W} R={R} {dt} state={st} same={same}")
    d = si.generate(wl)
    if same:
        d["qp"] = d["kp"].copy()
    dd = upload(d)
    state = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[st]
    core = make_core(dd, W, R, state)
    tok = [[dd[n][:, t:t + 1].contiguous().clone() for n in NAMES] for t in range(4)]
    # first token from M_0 (no continuation)
    y1, M1 = core.forward(*tok[0], variant=sdm.TIMEPAR)
    y2, M2 = core.forward(*tok[0], variant=sdm.TIMEPAR, staged=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(M1.view(torch.uint8), M2.view(torch.uint8))
    # three more tokens continuing the state
    for t in range(1, 4):
        y1, _ = core.forward(*tok[t], variant=sdm.TIMEPAR, M=M1, cont=True)
        y2, _ = core.forward(*tok[t], variant=sdm.TIMEPAR, M=M2, cont=True, staged=True)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"token {t}: y differs"
        assert torch.equal(M1.view(torch.uint8), M2.view(torch.uint8)), f"token {t}: M differs"
