"""Brute-force selection checker (numpy, float64).  TEST INFRASTRUCTURE ONLY.

Independent of `sdm_oracle.c`: it materialises all N = sqrtN^2 outer-sum
scores of a pre-PKM vector and sorts them, which is the plain definition of
"the top-K slots" that the two-stage product-key method must reproduce
[explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量", §3.1 step 1;
"Technical Summary: Sparse Delta Memory (SDM)", Core Mechanism item 2].
Order: exact score descending, then flat index n = i*sqrtN + j ascending.
Only meant for tiny N or a few sampled vectors.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns, widened exactly
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float64)


def scores(x: np.ndarray, sqrtN: int):
    """All N exact scores of one vector as (hi, lo) float64 arrays of length N."""
    x = _as_f64(x).reshape(-1)
    assert x.shape[0] == 2 * sqrtN
    a = np.repeat(x[:sqrtN], sqrtN)      # k'_1[i] for n = i*sqrtN + j
    b = np.tile(x[sqrtN:], sqrtN)        # k'_2[j]
    hi = a + b
    bv = hi - a
    lo = (a - (hi - bv)) + (b - bv)      # TwoSum error term: hi + lo == a + b
    return hi, lo


def topk(x: np.ndarray, sqrtN: int, K: int):
    """(idx int32 [K], w float64 [K]) for one vector, by sorting all N scores."""
    hi, lo = scores(x, sqrtN)
    n = np.arange(sqrtN * sqrtN)
    order = np.lexsort((n, -lo, -hi))[:K]
    d = (hi[order] - hi[order[0]]) + (lo[order] - lo[order[0]])
    e = np.exp(d)
    return order.astype(np.int32), e / e.sum()


def topk_rows(x: np.ndarray, sqrtN: int, K: int):
    """topk over the leading dims of x[..., 2*sqrtN]."""
    x = np.asarray(x)
    lead = x.shape[:-1]
    flat = x.reshape(-1, x.shape[-1])
    idx = np.empty((flat.shape[0], K), dtype=np.int32)
    w = np.empty((flat.shape[0], K), dtype=np.float64)
    for r in range(flat.shape[0]):
        idx[r], w[r] = topk(flat[r], sqrtN, K)
    return idx.reshape(lead + (K,)), w.reshape(lead + (K,))
