"""Seeded synthetic inputs for the SDM recurrent core.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random tensors following the workload recipe below;
it contains none of the method's arithmetic (no scores, no selection, no state
update), so both sides of a parity check can take their inputs from it.

Recipe (the same for every workload shape):
  * k', q'  ~ N(0, 1)                    shape [B, T, H, 2*sqrtN]
  * v       ~ N(0, 1)                    shape [B, T, H, d_v]
  * alpha   = exp(-A_h * softplus(u)),   A_h ~ U[1, 16] per head, u ~ N(-4, 1)
                                          per (b, t, h)  -> shape [B, T, H]
  * beta    = sigmoid(z),                z ~ N(0, 1) per (b, t, h)
  * M_0     ~ N(0, 0.02^2)               shape [H, N, d_v], N = sqrtN^2
  * optional key reuse: for every (b, t) with t >= 1, with probability
    `reuse` the whole k'[b, t, :, :] (all heads) is replaced by
    k'[b, t', :, :] with t' uniform in {0, ..., t-1}; rows are filled in t
    order, so a copied row may itself be a copy.  q' and v are never reused.
Values are drawn in float64, rounded to float32 (round to nearest even) and,
for the bf16 workloads, rounded once more to bfloat16 (round to nearest even);
bf16 tensors are returned as uint16 bit patterns.  alpha and beta are
evaluated in float64 from the float32-rounded u and z (A_h stays float64),
then rounded to float32.

Bits are independent of the thread count: every tensor gets its own child of
SeedSequence(seed), and every (b, 1024-token block) of it, or (head, 4096-slot
block) of M_0, gets its own grandchild stream.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

T_BLOCK = 1024  # token block that owns one random stream (part of the recipe)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    sqrtN: int
    d_v: int
    W: int
    R: int
    dtype: str  # dtype of k', q', v: "f32" or "bf16"
    reuse: float
    seed: int

    @property
    def N(self) -> int:
        return self.sqrtN * self.sqrtN

    @property
    def head_tokens(self) -> int:
        return self.B * self.T * self.H

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five synthetic workloads.  Sizes follow the isoFLOP shapes on the pages:
# W = R = d_qk of the dense baseline (64), head count H sets the state size.
WORKLOADS = {
    0: Workload("tiny", B=1, T=64, H=1, sqrtN=16, d_v=32, W=4, R=4,
                dtype="f32", reuse=0.0, seed=1000),
    1: Workload("1.4B-style layer", B=8, T=4096, H=4, sqrtN=128, d_v=512,
                W=64, R=64, dtype="f32", reuse=0.0, seed=1001),
    2: Workload("larger state", B=4, T=16384, H=2, sqrtN=256, d_v=1024,
                W=64, R=64, dtype="f32", reuse=0.1, seed=1002),
    3: Workload("8B-style layer", B=8, T=8192, H=4, sqrtN=256, d_v=1024,
                W=64, R=64, dtype="f32", reuse=0.0, seed=1003),
    4: Workload("long-context single sequence", B=1, T=1 << 20, H=1,
                sqrtN=512, d_v=2048, W=64, R=64, dtype="bf16", reuse=0.1,
                seed=1004),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads(threads):
    if threads is not None:
        return max(1, int(threads))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _child(ss: np.random.SeedSequence, *key) -> np.random.SeedSequence:
    """The stream of sub-block `key` of tensor stream `ss` (stateless)."""
    return np.random.SeedSequence(ss.entropy, spawn_key=tuple(ss.spawn_key) + key)


def _normal_blocks(ss: np.random.SeedSequence, B, T, inner, scale, loc, out_dtype,
                   pool) -> np.ndarray:
    """Draw N(loc, scale^2) of shape [B, T, *inner]; one stream per (b, block)."""
    inner = tuple(inner)
    nblk = (T + T_BLOCK - 1) // T_BLOCK
    if out_dtype == "bf16":
        out = np.empty((B, T) + inner, dtype=np.uint16)
    else:
        out = np.empty((B, T) + inner, dtype=np.float32)

    def job(i):
        b, k = divmod(i, nblk)
        t0 = k * T_BLOCK
        t1 = min(T, t0 + T_BLOCK)
        g = np.random.Generator(np.random.PCG64(_child(ss, b, k)))
        x = g.standard_normal(size=(t1 - t0,) + inner)
        if scale != 1.0 or loc != 0.0:
            x = x * scale + loc
        x32 = x.astype(np.float32)
        out[b, t0:t1] = f32_to_bf16_bits(x32) if out_dtype == "bf16" else x32

    list(pool.map(job, range(B * nblk)))
    return out


def _reuse_sources(ss: np.random.SeedSequence, B, T, p) -> np.ndarray:
    """For each (b, t) the token whose k' row ends up at t (t itself if no reuse)."""
    src = np.tile(np.arange(T, dtype=np.int64), (B, 1))
    if p <= 0.0 or T < 2:
        return src
    g = np.random.Generator(np.random.PCG64(ss))
    for b in range(B):
        hit = g.random(T) < p
        u = g.random(T)
        hit[0] = False
        tt = np.nonzero(hit)[0]
        # t' uniform in {0..t-1}
        tp = np.minimum((u[tt] * tt).astype(np.int64), tt - 1)
        row = src[b]
        # fill in t order: a reused row copies the (already final) source row
        for t, s in zip(tt.tolist(), tp.tolist()):
            row[t] = row[s]
    return src


def generate(wl: Workload, T: int | None = None, threads: int | None = None) -> dict:
    """Inputs for workload `wl` (optionally truncated to its first T tokens).

    Returns a dict with kp, qp, v ([B,T,H,*], float32 or uint16 bf16 bits),
    alpha, beta ([B,T,H] float32), M0 ([H,N,d_v] float32) and the key-reuse
    source map `src` ([B,T] int64).
    """
    T = wl.T if T is None else int(T)
    B, H, S, D = wl.B, wl.H, wl.sqrtN, wl.d_v
    root = np.random.SeedSequence(wl.seed)
    s_k, s_q, s_v, s_a, s_u, s_z, s_m, s_r = root.spawn(8)
    with ThreadPoolExecutor(_threads(threads)) as pool:
        kp = _normal_blocks(s_k, B, T, (H, 2 * S), 1.0, 0.0, wl.dtype, pool)
        qp = _normal_blocks(s_q, B, T, (H, 2 * S), 1.0, 0.0, wl.dtype, pool)
        v = _normal_blocks(s_v, B, T, (H, D), 1.0, 0.0, wl.dtype, pool)
        u = _normal_blocks(s_u, B, T, (H,), 1.0, -4.0, "f32", pool)
        z = _normal_blocks(s_z, B, T, (H,), 1.0, 0.0, "f32", pool)
        # M_0: one stream per (head, block of 4096 slots)
        N = S * S
        M0 = np.empty((H, N, D), dtype=np.float32)
        nb = (N + 4095) // 4096

        def mjob(i):
            h, k = divmod(i, nb)
            n0, n1 = k * 4096, min(N, (k + 1) * 4096)
            g = np.random.Generator(np.random.PCG64(_child(s_m, h, k)))
            M0[h, n0:n1] = (g.standard_normal(size=(n1 - n0, D)) * 0.02).astype(np.float32)

        list(pool.map(mjob, range(H * nb)))
    A = np.random.Generator(np.random.PCG64(s_a)).uniform(1.0, 16.0, size=H)
    u64 = u.astype(np.float64)
    softplus = np.logaddexp(0.0, u64)
    alpha = np.exp(-A[None, None, :] * softplus).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    src = _reuse_sources(s_r, B, T, wl.reuse)
    if wl.reuse > 0.0:
        for b in range(B):
            if not np.array_equal(src[b], np.arange(T)):
                kp[b] = kp[b][src[b]]
    return dict(kp=kp, qp=qp, v=v, alpha=alpha, beta=beta, M0=M0, src=src)


def as_f32(x: np.ndarray) -> np.ndarray:
    """float32 view of an input tensor (bf16 bit patterns are widened exactly)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)
