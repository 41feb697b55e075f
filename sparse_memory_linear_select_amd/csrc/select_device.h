// Building blocks of the product-key top-K selection shared by the
// selection kernels and the one-token kernel (see select.hip for the method
// and the explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量",
// §3.1 step 1, and "Technical Summary: Sparse Delta Memory (SDM)", Core
// Mechanism 2, for the identity it rests on).  Keys are 64-bit: the
// order-preserving bits of a value above its inverted index (stage 1), or of
// the TwoSum pair hi : lo of a pair's exact score (stage 2).
#pragma once

#include "lane_ops.h"

namespace sdm {
namespace {

constexpr int kTabMax = 320;  // >= number of pruned pairs for K = 64 (280)

__device__ __forceinline__ uint32_t f2ord(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;  // -0 and +0 are the same score
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float ord2f(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint32_t shl(uint32_t v, int src)
{
    return (uint32_t)__shfl((int)v, src, 64);
}

__device__ __forceinline__ uint64_t shl64(uint64_t v, int src)
{
    const uint32_t lo = shl((uint32_t)v, src), hi = shl((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t dpp_xor64(uint64_t v, int m)
{
    return ((uint64_t)dpp_xor((uint32_t)(v >> 32), m) << 32) | dpp_xor((uint32_t)v, m);
}

__device__ __forceinline__ void pair_vals64(uint64_t v, int m, uint64_t &lo, uint64_t &hi)
{
    uint32_t l0, h0, l1, h1;
    pair_vals((uint32_t)v, m, l0, h0);
    pair_vals((uint32_t)(v >> 32), m, l1, h1);
    lo = ((uint64_t)l1 << 32) | l0;
    hi = ((uint64_t)h1 << 32) | h0;
}

// This lane's key after a compare-exchange with lane ^ m: the larger key of
// the pair if keep_max, else the smaller (one compare; equal keys: either).
__device__ __forceinline__ uint64_t xchg_max(uint64_t k, int m, bool keep_max)
{
    if (m >= 16) {
        uint64_t lo, hi;
        pair_vals64(k, m, lo, hi);
        return ((lo > hi) == keep_max) ? lo : hi;
    }
    const uint64_t o = dpp_xor64(k, m);
    return ((o > k) == keep_max) ? o : k;
}

// Orders LDS traffic between the lanes of one wavefront.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void two_sum(float a, float b, float &s, float &e)
{
    s = a + b;
    const float bv = s - a;
    const float av = s - bv;
    e = (a - av) + (b - bv);
}

__device__ __forceinline__ float load_elem(const void *x, bool bf16, int64_t i)
{
    if (bf16) return __uint_as_float((uint32_t)((const uint16_t *)x)[i] << 16);
    return ((const float *)x)[i];
}

// Step (KK, J) of the bitonic network (descending) over NA arrays of 64*E
// keys each, element e = lane*E + r; the steps are instantiated one by one
// so that every lane pattern is a compile-time constant (the DPP controls
// must be immediates).
template <int NA, int E, int KK, int J>
__device__ __forceinline__ void sort_step(uint64_t (&k)[NA][E], int lane)
{
    if constexpr (J < E) {  // partner in the same lane
#pragma unroll
        for (int r = 0; r < E; r++) {
            if ((r & J) == 0) {
                // one compare per exchange: swap when the pair is out of the
                // step's direction (equal keys: either way)
                const int e = lane * E + r;
                const bool desc = (e & KK) == 0;
#pragma unroll
                for (int i = 0; i < NA; i++) {
                    const uint64_t a = k[i][r], b = k[i][r | J];
                    const bool sw = (a < b) == desc;
                    k[i][r] = sw ? b : a;
                    k[i][r | J] = sw ? a : b;
                }
            }
        }
    } else {  // partner in lane ^ (J / E), same register
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            const bool keep_max = ((e & J) == 0) == ((e & KK) == 0);
#pragma unroll
            for (int i = 0; i < NA; i++) k[i][r] = xchg_max(k[i][r], J / E, keep_max);
        }
    }
}

template <int NA, int E, int KK, int J>
__device__ __forceinline__ void sort_steps(uint64_t (&k)[NA][E], int lane)
{
    sort_step<NA, E, KK, J>(k, lane);
    if constexpr (J > 1) sort_steps<NA, E, KK, J / 2>(k, lane);
}

template <int NA, int E, int KK>
__device__ __forceinline__ void sort_stages(uint64_t (&k)[NA][E], int lane)
{
    sort_steps<NA, E, KK, KK / 2>(k, lane);
    if constexpr (KK < 64 * E) sort_stages<NA, E, 2 * KK>(k, lane);
}

// Sort each of NA arrays of 64*E keys, descending; element e = lane*E + r.
template <int NA, int E>
__device__ __forceinline__ void sort_desc(uint64_t (&k)[NA][E], int lane)
{
    sort_stages<NA, E, 2>(k, lane);
}

// Does candidate (ka, na) come before (kb, nb)?  Higher exact score first,
// then lower flat slot index.
__device__ __forceinline__ bool before(uint64_t ka, uint32_t na, uint64_t kb, uint32_t nb)
{
    return ka > kb || (ka == kb && na < nb);
}

// Compare-exchange of (k, n) with lane ^ m: this lane keeps the entry of the
// pair that comes first if keep_first, else the other one.
__device__ __forceinline__ void ce_lane(uint64_t &k, uint32_t &n, int m, bool keep_first)
{
    if (m >= 16) {
        uint64_t lk, uk;
        uint32_t ln, un;
        pair_vals64(k, m, lk, uk);
        pair_vals(n, m, ln, un);
        const bool take_lo = before(lk, ln, uk, un) == keep_first;
        k = take_lo ? lk : uk;
        n = take_lo ? ln : un;
        return;
    }
    const uint64_t ok = dpp_xor64(k, m);
    const uint32_t on = dpp_xor(n, m);
    const bool take = before(k, n, ok, on) != keep_first;
    k = take ? ok : k;  // selects, not a branch on the lane mask
    n = take ? on : n;
}

// Sort one 64-entry column (one entry per lane) in canonical order.
template <int KK, int J>
__device__ __forceinline__ void col_sort_steps(uint64_t &k, uint32_t &n, int lane)
{
    ce_lane(k, n, J, ((lane & J) == 0) == ((lane & KK) == 0));
    if constexpr (J > 1) col_sort_steps<KK, J / 2>(k, n, lane);
}

template <int KK>
__device__ __forceinline__ void col_sort_stages(uint64_t &k, uint32_t &n, int lane)
{
    col_sort_steps<KK, KK / 2>(k, n, lane);
    if constexpr (KK < 64) col_sort_stages<2 * KK>(k, n, lane);
}

// Bitonic clean-up of one 64-entry column: steps 32, 16, ..., 1.
template <int J>
__device__ __forceinline__ void col_clean(uint64_t &k, uint32_t &n, int lane)
{
    ce_lane(k, n, J, (lane & J) == 0);
    if constexpr (J > 1) col_clean<J / 2>(k, n, lane);
}

__device__ __forceinline__ void col_sort(uint64_t &k, uint32_t &n, int lane)
{
    col_sort_stages<2>(k, n, lane);
}

// (ka, na) <- first 64 of two sorted columns, sorted.
// (ka, na) <- first 64 of a sorted column and of a sorted column given
// reversed (lane l holds its entry 63 - l), sorted.
__device__ __forceinline__ void col_merge_rev(uint64_t &ka, uint32_t &na, uint64_t rk, uint32_t rn,
                                              int lane)
{
    if (!before(ka, na, rk, rn)) {
        ka = rk;
        na = rn;
    }
    col_clean<32>(ka, na, lane);
}

__device__ __forceinline__ void col_merge(uint64_t &ka, uint32_t &na, uint64_t kb, uint32_t nb,
                                          int lane)
{
    col_merge_rev(ka, na, shl64(kb, 63 - lane), shl(nb, 63 - lane), lane);
}

// Sort one 64-entry bitonic column (falling, then rising) in canonical order.
__device__ __forceinline__ void col_bitonic(uint64_t &k, uint32_t &n, int lane)
{
    col_clean<32>(k, n, lane);
}

// Pair of per-half ranks (a << 8 | b) held by `lane` in candidate column `col`
// for a list of K, or kNoPair.  The pruned pairs (a+1)(b+1) <= K split into
// hooks h = min(a, b): row part (h, b >= h) and column part (a > h, h), each
// already in canonical order (scores fall along a row and down a column,
// ties keep the lower index first).  Columns:
//   0  (0, b), b < K                               sorted
//   1  (a, 0), 1 <= a < K                          sorted
//   2  hook 1: row part from lane 0 up, column
//      part from lane 63 down                      bitonic
//   3, 4  hooks h >= 2, concatenated               unsorted
constexpr uint16_t kNoPair = 0xFFFF;

__host__ __device__ inline uint16_t hook_pair(int K, int col, int lane)
{
    if (col == 0) return lane < K ? (uint16_t)lane : kNoPair;
    if (col == 1) return lane + 1 < K ? (uint16_t)((lane + 1) << 8) : kNoPair;
    if (col == 2) {
        const int end = K / 2;  // hook 1 spans ranks 1 .. end-1
        if (lane + 1 < end) return (uint16_t)((1 << 8) | (lane + 1));
        const int a = 2 + (63 - lane);
        if (lane > 63 - (end - 2) && a < end) return (uint16_t)((a << 8) | 1);
        return kNoPair;
    }
    int idx = (col - 3) * 64 + lane;
    for (int h = 2; (h + 1) * (h + 1) <= K; h++) {
        const int end = K / (h + 1);
        const int nr = end - h, nc = end - h - 1;
        if (idx < nr) return (uint16_t)((h << 8) | (h + idx));
        idx -= nr;
        if (idx < nc) return (uint16_t)(((h + 1 + idx) << 8) | h);
        idx -= nc;
    }
    return kNoPair;
}

// Number of pruned pairs with both ranks >= 2 (columns 3 and 4).
__host__ __device__ inline int hook_rest(int K)
{
    int n = 0;
    for (int h = 2; (h + 1) * (h + 1) <= K; h++) n += 2 * (K / (h + 1) - h) - 1;
    return n;
}

// Candidate pair ab = a << 8 | b of ranks (or kNoPair: the empty entry, after
// every real candidate): its exact score key and flat slot, from the halves'
// first entries in LDS (see select_pairs).
__device__ __forceinline__ void pair_entry(const float *v1, const float *v2, const uint32_t *i1,
                                           const uint32_t *i2, uint32_t ab, int S, uint64_t &k,
                                           uint32_t &n)
{
    k = 0;
    n = 0xFFFFFFFFu;
    if (ab != kNoPair) {
        const int ra = (int)(ab >> 8), rb = (int)(ab & 0xFF);
        float hi, lo;
        two_sum(v1[ra], v2[rb], hi, lo);
        k = ((uint64_t)f2ord(hi) << 32) | f2ord(lo);
        n = i1[ra] * (uint32_t)S + i2[rb];
    }
}

// Stage 2 of one list of K <= 64 slots, from the first K entries of each
// half in rank order (values v1[a], v2[b] and half indices i1[a], i2[b] in
// LDS private to the wavefront, visible to all its lanes).  Lane l < K
// returns the l-th selected pair in canonical order: its exact score key
// (TwoSum hi : lo, order-preserving bits) and flat slot n = i1*sqrtN + i2.
// v1, v2 and i1 serve as scratch once their entries are read.
template <int E2>
__device__ __forceinline__ void select_pairs(float *v1, float *v2, uint32_t *i1, const uint32_t *i2,
                                             const uint16_t (&tabv)[E2], int K, int rest, int S,
                                             int lane, uint64_t &key_out, uint32_t &n_out)
{
    // ---- stage 2: exact sums of the pruned rank pairs ----
    uint64_t ck[E2];
    uint32_t cn[E2];
#pragma unroll
    for (int r = 0; r < E2; r++) pair_entry(v1, v2, i1, i2, tabv[r], S, ck[r], cn[r]);
    // columns 0, 1 sorted; 2 bitonic; 3, 4 unsorted (K-uniform branches)
    if (K >= 2) col_merge(ck[0], cn[0], ck[1], cn[1], lane);
    if (K >= 4) {
        col_bitonic(ck[2], cn[2], lane);
        col_merge(ck[0], cn[0], ck[2], cn[2], lane);
    }
    if (rest > 0) {
        // Columns 0-2 now hold the first 64 of hooks 0 and 1, sorted.  A
        // pair of hooks >= 2 that does not come before its K-th entry has
        // K pairs before it and cannot be selected; the others (about 20
        // of 92 for Gaussian scores) are compacted into one column.
        const uint64_t tk = shl64(ck[0], K - 1);
        const uint32_t tn = shl(cn[0], K - 1);
        const bool s3 = before(ck[3], cn[3], tk, tn);
        const bool s4 = (rest > 64) && before(ck[4], cn[4], tk, tn);
        const uint64_t m3 = __ballot(s3), m4 = __ballot(s4);
        const int n3 = __popcll(m3), tot = n3 + __popcll(m4);
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int r3 = __popcll(m3 & below), r4 = n3 + __popcll(m4 & below);
        uint32_t *xh = reinterpret_cast<uint32_t *>(v1);
        uint32_t *xl = reinterpret_cast<uint32_t *>(v2);
        uint32_t *xn = i1;
        // 64 survivors at a time (more than 64 is rare)
        for (int base = 0; base < tot; base += 64) {
            wave_sync();  // earlier reads of v1, v2 and i1 are done
            if (s3 & (r3 >= base) & (r3 < base + 64)) {
                xh[r3 - base] = (uint32_t)(ck[3] >> 32);
                xl[r3 - base] = (uint32_t)ck[3];
                xn[r3 - base] = cn[3];
            }
            if (s4 & (r4 >= base) & (r4 < base + 64)) {
                xh[r4 - base] = (uint32_t)(ck[4] >> 32);
                xl[r4 - base] = (uint32_t)ck[4];
                xn[r4 - base] = cn[4];
            }
            wave_sync();
            uint64_t sk = 0;
            uint32_t sn = 0xFFFFFFFFu;
            if (lane < tot - base) {
                sk = ((uint64_t)xh[lane] << 32) | xl[lane];
                sn = xn[lane];
            }
            col_sort(sk, sn, lane);
            col_merge(ck[0], cn[0], sk, sn, lane);
        }
    }
    key_out = ck[0];
    n_out = cn[0];
}

// Softmax weight of lane l's selected score (0 for l >= K); lane 0 holds the
// largest score.
__device__ __forceinline__ float select_weight(uint64_t key, int K, int lane)
{
    const float hi = ord2f((uint32_t)(key >> 32));
    const float lo = ord2f((uint32_t)key);
    const float hi0 = __builtin_amdgcn_readfirstlane(hi);  // every lane is active here
    const float lo0 = __builtin_amdgcn_readfirstlane(lo);
    const float ex = lane < K ? expf((hi - hi0) + (lo - lo0)) : 0.0f;
    float z = ex;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z = xor_add(z, o);
    return ex / z;
}

}  // namespace
}  // namespace sdm
