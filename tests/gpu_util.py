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
# for |ref| ~ 1.  The GPU rounds its float32 result, the oracle its float64
# result, to bfloat16: they differ by one spacing (2^-8 relative) where the
# two straddle a rounding boundary (chance ~2^-15 per stored value), and
# reads that see a write of the same epoch skip that write's rounding (at
# most half a spacing); writes are contractions, so such differences shrink.
TOL_BF16 = 2.0 ** -7


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def upload(d: dict) -> dict:
    return {k: to_dev(v) for k, v in d.items() if k != "src"}


def make_core(dd: dict, W: int, R: int, state=torch.float32) -> sdm.SDM:
    return sdm.SDM(dd["M0"], W, R, state=state)


def gpu_forward(d: dict, W: int, R: int, variant=sdm.AUTO, state=torch.float32):
    dd = upload(d)
    core = make_core(dd, W, R, state)
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
