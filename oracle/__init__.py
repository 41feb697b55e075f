"""Float64 CPU oracle for the SDM recurrent core.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (the C source is `sdm_oracle.c` in this
directory, compiled with gcc).

Functions
---------
select(x, sqrtN, K, dtype)      -> idx [..., K] int32, w [..., K] float64
forward(inp, wl, c0, c1)        -> dict(Iw, kw, Ir, qw, y, M) (float64 y, M)
recurrence(sel, inp, wl, c0, c1)-> (y, M) from a given selection

See `sdm_oracle.c` for what each step computes and which passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdm_oracle.c")
_LIB = os.path.join(_HERE, "libsdm_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (float64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            p = ctypes.c_void_p
            lib.sdm_oracle_topk_rows.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                 p, ctypes.c_int, p, p, p, p, ctypes.c_int]
            lib.sdm_oracle_topk_rows.restype = ctypes.c_int
            lib.sdm_oracle_recurrence.argtypes = [
                ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, p, p, p, p, p, ctypes.c_int, p, p, p,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, p, p, ctypes.c_int]
            lib.sdm_oracle_recurrence.restype = ctypes.c_int
            lib.sdm_oracle_backward.argtypes = [
                ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, p, p, p, p, p, ctypes.c_int, p, p, p, p, p,
                p, p, p, p, p, p, ctypes.c_int]
            lib.sdm_oracle_backward.restype = ctypes.c_int
            lib.sdm_oracle_round_bf16.argtypes = [p, p, ctypes.c_int64]
            lib.sdm_oracle_round_bf16.restype = None
            lib.sdm_oracle_round_fp8.argtypes = [p, p, ctypes.c_int64, ctypes.c_int]
            lib.sdm_oracle_round_fp8.restype = None
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are float32 or bf16 bits (uint16), got {a.dtype}")


def select(x: np.ndarray, sqrtN: int, K: int, threads: int | None = None,
           scores: bool = False):
    """Top-K slots of each pre-PKM vector in x[..., 2*sqrtN].

    Returns (idx int32 [..., K], w float64 [..., K]) and, with scores=True,
    also the exact scores as float64 pairs (hi, lo).
    """
    x = np.ascontiguousarray(x)
    if x.shape[-1] != 2 * sqrtN:
        raise ValueError("last dim must be 2*sqrtN")
    lead = x.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    idx = np.empty(lead + (K,), dtype=np.int32)
    w = np.empty(lead + (K,), dtype=np.float64)
    hi = np.empty(lead + (K,), dtype=np.float64) if scores else None
    lo = np.empty(lead + (K,), dtype=np.float64) if scores else None
    rc = _load().sdm_oracle_topk_rows(
        rows, sqrtN, K, _ptr(x), _dtype_code(x), _ptr(idx), _ptr(w),
        _ptr(hi) if scores else None, _ptr(lo) if scores else None,
        threads or default_threads())
    if rc != 0:
        raise ValueError(f"sdm_oracle_topk_rows failed ({rc})")
    return (idx, w, hi, lo) if scores else (idx, w)


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 values (ties to even) of float64 x, as float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().sdm_oracle_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def round_fp8(x, scale_log2: int = 0) -> np.ndarray:
    """Nearest values of the E4M3 format scaled by 2^scale_log2 (ties to even,
    saturated at +-448 * 2^scale_log2), as float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().sdm_oracle_round_fp8(_ptr(x), _ptr(out), x.size, int(scale_log2))
    return out


STATE_MODES = {"f32": 0, "bf16": 1, "fp8": 2}


def recurrence(Iw, kw, Ir, qw, v, alpha, beta, M0, sqrtN: int, c0: int = 0,
               c1: int | None = None, threads: int | None = None, state: str = "f32",
               scale_log2: int = 0):
    """Token-serial write/read from a given selection; columns [c0, c1).
    state="bf16" holds the state in bfloat16, state="fp8" in E4M3 scaled by
    2^scale_log2 (rounded at init and after every write)."""
    assert state in STATE_MODES
    B, T, H, W = Iw.shape
    R = Ir.shape[-1]
    d_v = v.shape[-1]
    c1 = d_v if c1 is None else c1
    N = sqrtN * sqrtN
    nc = c1 - c0
    arrs = [np.ascontiguousarray(a) for a in (Iw, kw, Ir, qw, v, alpha, beta, M0)]
    Iw, kw, Ir, qw, v, alpha, beta, M0 = arrs
    assert Iw.dtype == np.int32 and Ir.dtype == np.int32
    assert kw.dtype == np.float64 and qw.dtype == np.float64
    assert alpha.dtype == np.float32 and beta.dtype == np.float32 and M0.dtype == np.float32
    assert M0.shape == (H, N, d_v)
    y = np.empty((B, T, H, nc), dtype=np.float64)
    M = np.empty((B, H, N, nc), dtype=np.float64)
    rc = _load().sdm_oracle_recurrence(
        B, T, H, sqrtN, d_v, W, R, _ptr(Iw), _ptr(kw), _ptr(Ir), _ptr(qw), _ptr(v),
        _dtype_code(v), _ptr(alpha), _ptr(beta), _ptr(M0), STATE_MODES[state], int(scale_log2),
        c0, c1, _ptr(y), _ptr(M), threads or default_threads())
    if rc != 0:
        raise ValueError(f"sdm_oracle_recurrence failed ({rc})")
    return y, M


def forward(inp: dict, sqrtN: int, W: int, R: int, c0: int = 0, c1: int | None = None,
            threads: int | None = None, state: str = "f32", scale_log2: int = 0) -> dict:
    """Selection plus recurrence on the inputs of `sdm_inputs.generate`."""
    Iw, kw = select(inp["kp"], sqrtN, W, threads)
    Ir, qw = select(inp["qp"], sqrtN, R, threads)
    y, M = recurrence(Iw, kw, Ir, qw, inp["v"], inp["alpha"], inp["beta"], inp["M0"],
                      sqrtN, c0, c1, threads, state, scale_log2)
    return dict(Iw=Iw, kw=kw, Ir=Ir, qw=qw, y=y, M=M)


def backward(inp: dict, sqrtN: int, W: int, R: int, dy, dMT=None,
             threads: int | None = None) -> dict:
    """Gradients of the core (float64 state, selections held fixed) for the
    upstream gradients dy [B,T,H,d_v] and dMT [B,H,N,d_v] (None: zero).
    Returns dkp, dqp [B,T,H,2 sqrtN], dv [B,T,H,d_v], dalpha, dbeta [B,T,H]
    and dM0 [H,N,d_v], all float64."""
    Iw, kw = select(inp["kp"], sqrtN, W, threads)
    Ir, qw = select(inp["qp"], sqrtN, R, threads)
    v, alpha, beta, M0 = (np.ascontiguousarray(inp[k]) for k in ("v", "alpha", "beta", "M0"))
    B, T, H, d_v = v.shape
    N = sqrtN * sqrtN
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    assert dy.shape == (B, T, H, d_v)
    if dMT is not None:
        dMT = np.ascontiguousarray(dMT, dtype=np.float64)
        assert dMT.shape == (B, H, N, d_v)
    out = dict(dkp=np.empty((B, T, H, 2 * sqrtN)), dqp=np.empty((B, T, H, 2 * sqrtN)),
               dv=np.empty((B, T, H, d_v)), dalpha=np.empty((B, T, H)),
               dbeta=np.empty((B, T, H)), dM0=np.empty((H, N, d_v)))
    rc = _load().sdm_oracle_backward(
        B, T, H, sqrtN, d_v, W, R, _ptr(Iw), _ptr(kw), _ptr(Ir), _ptr(qw), _ptr(v),
        _dtype_code(v), _ptr(alpha), _ptr(beta), _ptr(M0), _ptr(dy),
        _ptr(dMT) if dMT is not None else None, _ptr(out["dkp"]), _ptr(out["dqp"]),
        _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dM0"]),
        threads or default_threads())
    if rc != 0:
        raise ValueError(f"sdm_oracle_backward failed ({rc})")
    return out
