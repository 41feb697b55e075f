"""Helpers shared by the GPU parity tests (inputs -> device, oracle comparison)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm

TOL = 1e-4       # max |gpu - ref| <= TOL * (1 + |ref|) for y and M
TOL_LONG = 1e-3  # the same bound for the 2^20-token sequence
WTOL = 1e-5      # absolute bound on the softmax weights (diagnostic)
# bfloat16 state: the same form of bound at 2^-7, i.e. two bfloat16 spacings
# for |ref| ~ 1, as the outer bound.  The GPU rounds its float32 result, the
# oracle its float64 result, to bfloat16: they differ by one spacing (2^-8
# relative) only where the two straddle a rounding boundary (chance ~2^-15
# per stored value); writes are contractions, so such differences shrink.
# Everywhere else both hold the same bits, which the bfloat16 tests check
# through the fraction of elements within TOL.
TOL_BF16 = 2.0 ** -7
# E4M3 state: the same outer bound at 2^-2, two E4M3 spacings (3 mantissa
# bits) at |ref| ~ 1, for the same reason.
TOL_FP8 = 2.0 ** -2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def upload(d: dict) -> dict:
    return {k: to_dev(v) for k, v in d.items() if k != "src"}


FP8_SCALE_LOG2 = -4  # E4M3 state scale used by the tests: codes of M * 2^4


def make_core(dd: dict, W: int, R: int, state=torch.float32, scale_log2=FP8_SCALE_LOG2) -> sdm.SDM:
    return sdm.SDM(dd["M0"], W, R, state=state, state_scale_log2=scale_log2)


def gpu_forward(d: dict, W: int, R: int, variant=sdm.AUTO, state=torch.float32,
                scale_log2=FP8_SCALE_LOG2):
    dd = upload(d)
    core = make_core(dd, W, R, state, scale_log2)
    y, M = core.forward(dd["kp"], dd["qp"], dd["v"], dd["alpha"], dd["beta"], variant=variant)
    torch.cuda.synchronize()
    return core, dd, y, M


def assert_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert worst <= tol, f"{what}: max |err|/(1+|ref|) = {worst:.3e} > {tol:.1e}"
    return worst


def check_selection(gI, gw, rI, rw, what: str):
    """Index lists bit-exact, weights within WTOL."""
    gI = np.asarray(gI).reshape(-1, np.shape(gI)[-1])
    rI = np.asarray(rI).reshape(-1, np.shape(rI)[-1])
    bad = np.nonzero((gI != rI).any(axis=-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} index lists differ (first rows {bad[:5]})"
    gw = np.asarray(gw, dtype=np.float64).reshape(gI.shape)
    werr = float(np.abs(gw - np.asarray(rw).reshape(gI.shape)).max()) if gw.size else 0.0
    assert werr <= WTOL, f"{what}: weight error {werr:.2e}"


class Timer:
    def __init__(self, name):
        self.name = name

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"  [{self.name}: {time.time() - self.t:.1f}s]")


def check_bf16_state(y, M, ref_y, ref_M, what="", outer=TOL_BF16):
    """GPU (bfloat16 or E4M3 state; M as values) vs the oracle's mode for the
    same state.  Outer bound: every element of y and M within
    outer * (1 + |ref|) (TOL_BF16, or TOL_FP8 for E4M3).  Inner bounds,
    which only reads of the stored, rounded rows meet: >= 99.99% of y within
    TOL * (1 + |ref|) and >= 99.9% of M equal to the oracle's bits (reading
    the unrounded composition of a slot's writes instead misses a rounding by
    up to half a bfloat16 spacing on every read that sees such a write).
    Returns (max rel err y, max rel err M, fraction of y within TOL, fraction
    of M equal)."""
    yg = np.asarray(y, dtype=np.float64)
    Mg = np.asarray(M, dtype=np.float64)
    fy = float((np.abs(yg - ref_y) <= TOL * (1.0 + np.abs(ref_y))).mean()) if yg.size else 1.0
    same = float((Mg == ref_M).mean()) if Mg.size else 1.0
    log(f"  {what}y within {TOL:.0e}: {fy:.6f}; M equal to the oracle's bits: {same:.6f}")
    ey = assert_close(yg, ref_y, outer, "y")
    eM = assert_close(Mg, ref_M, outer, "M")
    log(f"  {what}max rel err y {ey:.2e}  M {eM:.2e}")
    assert fy >= 0.9999, f"y: only {fy:.6f} of the elements within {TOL:.0e} * (1 + |ref|)"
    assert same >= 0.999, f"M: only {same:.6f} of the elements equal the oracle's"
    return ey, eM, fy, same

