"""GPU parity of sdm_select: index lists bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import check_selection, log, to_dev, Timer

pytestmark = pytest.mark.gpu


def _gpu_select(kp, qp, H, S, W, R, d_v=4):
    M0 = torch.zeros((H, S * S, d_v), dtype=torch.float32, device="cuda")
    core = sdm.SDM(M0, W, R)
    out = core.select(to_dev(kp), to_dev(qp))
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _compare(kp, qp, H, S, W, R, what, rows=None):
    Iw, kw, Ir, qw = _gpu_select(kp, qp, H, S, W, R)
    for x, K, gI, gw, nm in ((kp, W, Iw, kw, "write"), (qp, R, Ir, qw, "read")):
        flat = x.reshape(-1, 2 * S)
        gI2, gw2 = gI.reshape(-1, K), gw.reshape(-1, K)
        if rows is not None:
            flat, gI2, gw2 = flat[rows], gI2[rows], gw2[rows]
        rI, rw = oracle.select(flat, S, K)
        check_selection(gI2, gw2, rI, rw, f"{what} {nm}")
    return Iw, kw, Ir, qw


def test_select_tiny_workload():
    wl = si.WORKLOADS[0]
    log(f"select: {wl.name}")
    d = si.generate(wl)
    _compare(d["kp"], d["qp"], wl.H, wl.sqrtN, wl.W, wl.R, wl.name)


@pytest.mark.parametrize("S,W,R,dtype", [
    (1, 1, 1, "f32"), (2, 2, 1, "f32"), (13, 5, 13, "f32"), (64, 64, 64, "f32"),
    (65, 64, 7, "f32"), (100, 33, 48, "bf16"), (200, 64, 64, "f32"), (300, 17, 64, "bf16"),
    (700, 64, 64, "f32"), (1024, 64, 64, "bf16"),
])
def test_select_shapes(S, W, R, dtype):
    log(f"select: S={S} W={W} R={R} {dtype}")
    wl = si.Workload("shape", B=2, T=9, H=3, sqrtN=S, d_v=4, W=W, R=R, dtype=dtype,
                     reuse=0.0, seed=77 + S)
    d = si.generate(wl)
    _compare(d["kp"], d["qp"], wl.H, S, W, R, f"S={S}")


@pytest.mark.parametrize("S,K,span", [(8, 8, 2), (16, 16, 1), (64, 64, 3), (128, 64, 2)])
def test_select_massive_ties(S, K, span):
    """Small-integer inputs: most candidate scores tie exactly."""
    log(f"select ties: S={S} K={K}")
    rng = np.random.default_rng(S * 31 + K)
    kp = rng.integers(-span, span + 1, size=(1, 40, 2, 2 * S)).astype(np.float32)
    qp = np.where(rng.random(kp.shape) < 0.5, -0.0, 0.0).astype(np.float32)
    _compare(kp, qp, 2, S, K, K, "ties")


def test_select_extreme_magnitudes():
    """Exponent gaps of ~2^60 inside one sum: only an exact comparison orders them."""
    rng = np.random.default_rng(5)
    S = 32
    big = rng.choice([1.0, -1.0], size=(1, 64, 1, 2 * S)) * 2.0 ** 30
    tiny = rng.standard_normal((1, 64, 1, 2 * S)) * 2.0 ** -30
    kp = np.where(rng.random(big.shape) < 0.5, big, tiny).astype(np.float32)
    kp[..., S:] = np.where(rng.random((1, 64, 1, S)) < 0.5, big[..., S:] + tiny[..., S:], tiny[..., S:])
    _compare(kp.astype(np.float32), kp[:, ::-1].copy().astype(np.float32), 1, S, 16, 16, "extreme")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_select_full_workload(cfg):
    """All head-tokens of the workload on the GPU; the oracle checks a sample
    (all of them for the 1.4B-style layer)."""
    wl = si.WORKLOADS[cfg]
    log(f"select full: {wl.name}")
    with Timer("generate"):
        d = si.generate(wl)
    kp, qp = d["kp"], d["qp"]
    n = wl.head_tokens
    rows = None
    if cfg != 1:
        rows = np.sort(np.random.default_rng(cfg).choice(n, size=min(n, 16384), replace=False))
    with Timer("gpu + oracle"):
        Iw, kw, Ir, qw = _compare(kp, qp, wl.H, wl.sqrtN, wl.W, wl.R, wl.name, rows=rows)
    # every list, checked or not: distinct in-range slots, weights a distribution
    for I, w in ((Iw, kw), (Ir, qw)):
        s = np.sort(I, axis=-1)
        assert s.min() >= 0 and s.max() < wl.N and (np.diff(s, axis=-1) > 0).all()
        assert (w > 0).all() and np.abs(w.sum(-1) - 1).max() < 1e-5
        assert (np.diff(w, axis=-1) <= 1e-7).all()


@pytest.mark.parametrize("cfg,T", [(0, None), (1, 256), (4, 512)])
def test_write_histogram(cfg, T):
    """Write-slot utilisation counts per head equal the oracle's selection
    counted slot by slot; a second call accumulates."""
    wl = si.WORKLOADS[cfg]
    log(f"histogram: {wl.name} T={T or wl.T}")
    d = si.generate(wl, T=T)
    M0 = torch.zeros((wl.H, wl.N, 4), dtype=torch.float32, device="cuda")
    core = sdm.SDM(M0, wl.W, wl.R)
    kp = to_dev(d["kp"])
    counts = core.write_histogram(kp)
    torch.cuda.synchronize()
    Iw, _ = oracle.select(d["kp"], wl.sqrtN, wl.W)
    ref = np.stack([np.bincount(Iw[:, :, h].reshape(-1), minlength=wl.N) for h in range(wl.H)])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref)
    assert ref.sum() == wl.B * (T or wl.T) * wl.H * wl.W
    core.write_histogram(kp, counts)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(counts.cpu().numpy(), 2 * ref)
