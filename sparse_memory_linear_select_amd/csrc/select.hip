// Product-key top-K selection for the SDM core on gfx950.
//
// Per head-token and per list (k' -> W write slots, q' -> R read slots) one
// 64-lane wavefront:
//   stage 1  the two halves x_1 = x[0, sqrtN) and x_2 = x[sqrtN, 2 sqrtN) are
//            sorted in registers (bitonic network, lane-major layout, 64-bit
//            keys = order-preserving value bits : inverted index) and their
//            first K entries kept;
//   stage 2  candidate pairs (a, b) of per-half ranks with (a+1)(b+1) <= K are
//            scored with the exact sum x_1 + x_2 (TwoSum pair hi + lo in
//            float32, compared lexicographically = exact real order) and the
//            first K in the order (score desc, n = i*sqrtN + j asc) are kept.
//            The pairs are laid out in five 64-lane columns so that two
//            arrive sorted and one bitonic (runs along a row or down a
//            column of ranks are already in order); those three are merged
//            keeping the top 64, the pairs of the other two that do not come
//            before its K-th entry are dropped, and the survivors are
//            compacted into one column, sorted and merged in;
//   weights  softmax over the K selected scores.
// The compare-exchange steps form each list's dependent chain; their lane
// exchanges use DPP and the gfx950 permlane swaps (a few cycles) rather than
// the LDS crossbar.
// The product-key identity (select within each half first, then among sums of
// survivors) is stated in the explainer "Sparse Delta Memory：通过稀疏性扩展线性
// RNN 的状态容量", §3.1 step 1, and in "Technical Summary: Sparse Delta Memory
// (SDM)", Core Mechanism 2.  The pruning to (a+1)(b+1) <= K is exact: a pair
// of ranks (a, b) is preceded by every pair (a', b') with a' <= a, b' <= b
// (score at least as large, and on an equal score a smaller flat index), so
// with (a+1)(b+1) > K at least K pairs come before it.
#include "sdm_internal.h"

#include <array>
#include <cstring>

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

// Lane exchanges inside the compare-exchange networks.  These form the
// dependent chain of a selection, so they avoid the LDS crossbar
// (ds_bpermute):
//   m = 1, 2   one DPP quad permutation;
//   m = 4      row_shl:4 into banks 0 and 2 (lanes with bit 2 clear), then
//              row_shr:4 into banks 1 and 3 (bank = 4 lanes of a 16-lane row);
//   m = 8      row_ror:8 (a rotation by half of the 16-lane row);
//   m = 16, 32 the gfx950 permlane swaps, which give every lane both values
//              of its pair {l, l ^ m}: (lower lane's, upper lane's).
// m is a compile-time constant at every call (the networks are instantiated
// step by step); the DPP controls must be immediates, hence the switch.
__device__ __forceinline__ uint32_t dpp_xor(uint32_t x, int m)
{
    switch (m) {
    case 1: return __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false);
    case 4: {
        const uint32_t y = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x5, false);
        return __builtin_amdgcn_update_dpp(y, x, 0x114, 0xF, 0xA, false);
    }
    default: return __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xF, 0xF, false);
    }
}

__device__ __forceinline__ void pair_vals(uint32_t x, int m, uint32_t &lo, uint32_t &hi)
{
    if (m == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        lo = r[0];
        hi = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        lo = r[0];
        hi = r[1];
    }
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

// Step (KK, J) of the bitonic network over both halves (descending); the
// steps are instantiated one by one so that every lane pattern is a
// compile-time constant (the DPP controls must be immediates).
template <int E, int KK, int J>
__device__ __forceinline__ void sort_step(uint64_t (&k1)[E], uint64_t (&k2)[E], int lane)
{
    if constexpr (J < E) {  // partner in the same lane
#pragma unroll
        for (int r = 0; r < E; r++) {
            if ((r & J) == 0) {
                // one compare per exchange: swap when the pair is out of the
                // step's direction (equal keys: either way)
                const int e = lane * E + r;
                const bool desc = (e & KK) == 0;
                uint64_t a = k1[r], b = k1[r | J];
                bool sw = (a < b) == desc;
                k1[r] = sw ? b : a;
                k1[r | J] = sw ? a : b;
                a = k2[r];
                b = k2[r | J];
                sw = (a < b) == desc;
                k2[r] = sw ? b : a;
                k2[r | J] = sw ? a : b;
            }
        }
    } else {  // partner in lane ^ (J / E), same register
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            const bool keep_max = ((e & J) == 0) == ((e & KK) == 0);
            k1[r] = xchg_max(k1[r], J / E, keep_max);
            k2[r] = xchg_max(k2[r], J / E, keep_max);
        }
    }
}

template <int E, int KK, int J>
__device__ __forceinline__ void sort_steps(uint64_t (&k1)[E], uint64_t (&k2)[E], int lane)
{
    sort_step<E, KK, J>(k1, k2, lane);
    if constexpr (J > 1) sort_steps<E, KK, J / 2>(k1, k2, lane);
}

template <int E, int KK>
__device__ __forceinline__ void sort_stages(uint64_t (&k1)[E], uint64_t (&k2)[E], int lane)
{
    sort_steps<E, KK, KK / 2>(k1, k2, lane);
    if constexpr (KK < 64 * E) sort_stages<E, 2 * KK>(k1, k2, lane);
}

// Sort 64*E keys of each of two halves, descending; element e = lane*E + r.
template <int E>
__device__ __forceinline__ void sort_halves_desc(uint64_t (&k1)[E], uint64_t (&k2)[E], int lane)
{
    sort_stages<E, 2>(k1, k2, lane);
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
    const bool mine_first = before(k, n, ok, on);
    if (keep_first != mine_first) {
        k = ok;
        n = on;
    }
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
__device__ __forceinline__ void col_merge(uint64_t &ka, uint32_t &na, uint64_t kb, uint32_t nb,
                                          int lane)
{
    const uint64_t rk = shl64(kb, 63 - lane);
    const uint32_t rn = shl(nb, 63 - lane);
    if (!before(ka, na, rk, rn)) {
        ka = rk;
        na = rn;
    }
    col_clean<32>(ka, na, lane);
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

struct SelArgs {
    const void *kp, *qp;
    int bf16;
    int64_t T;
    int H, sqrtN, W, R;
    int64_t n_ht;   // head-tokens in the launch: B * tn * H
    int64_t t0, tn;  // token range [t0, t0 + tn) of every sequence
    int32_t *Iw, *Ir;
    float *kw, *qw;
    uint32_t *rec;
    int rec_dwords, Wp, Rp;
    const float *alpha, *beta;
    uint32_t *hist;  // [H][N] write-slot counts (histogram mode: write lists only)
    int lists;       // 2: write and read lists; 1: write lists only
    // state initialisation (SelInit): item i copies float4s [64 i, 64 i + 64)
    // of M0 to every sequence's slab of M (n4 float4s per slab)
    const float4 *M0;
    void *M;
    int64_t n4;
    int Bseq, init_bf16;
    // candidate columns of both lists (pairs a << 8 | b, laid out by hooks),
    // computed on the host: lane l of column c reads entry c*64 + l
    uint16_t tab[2][kTabMax];
    int tabn[2];  // pairs with both ranks >= 2 (columns 3 and 4)
};

template <int E, bool INIT>
__device__ __forceinline__ void select_body(SelArgs a)
{
    constexpr int E2 = 5;  // candidate columns: 5*64 >= 280 pairs for K = 64
    __shared__ float sv[4][2][64];
    __shared__ uint32_t si[4][2][64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const int S = a.sqrtN;
    // head-token arithmetic in 32 bits (B*T*H < 2^31) on wave-uniform values,
    // so that it runs on the scalar unit
    const uint32_t T32 = (uint32_t)a.T, H32 = (uint32_t)a.H;
    const uint32_t tn32 = (uint32_t)a.tn, t032 = (uint32_t)a.t0;
    const uint64_t items = (uint64_t)a.lists * (uint64_t)a.n_ht;  // < 2^32, but it + stride may not be
    // items alternate between the lists and the stride is even, so a wave
    // keeps one list: its candidate columns stay in registers
    const int list = a.lists == 2 ? (wv & 1) : 0;
    const int K = list ? a.R : a.W;
    const void *x = list ? a.qp : a.kp;
    const int rest = a.tabn[list];
    uint16_t tabv[E2];
#pragma unroll
    for (int r = 0; r < E2; r++) tabv[r] = a.tab[list][r * 64 + lane];
    for (uint64_t it = blockIdx.x * 4u + (uint32_t)wv; it < items; it += gridDim.x * 4u) {
        uint32_t ht = (uint32_t)(a.lists == 2 ? it >> 1 : it);
        if (tn32 != T32) {  // position in the token range -> (b*T + t)*H + h
            const uint32_t bb = ht / (tn32 * H32);
            ht += bb * (T32 - tn32) * H32 + t032 * H32;
        }
        const int64_t base = (int64_t)ht * 2 * S;
        // the gates of a write list, fetched now so their latency overlaps the selection
        float al = 0.0f, be = 0.0f;
        if (a.rec != nullptr && list == 0) {
            al = a.alpha[ht];
            be = a.beta[ht];
        }
        // this item's piece of M0, stored once the stage-1 sort is done
        const int64_t jm = (int64_t)it * 64 + lane;
        const bool init = INIT && jm < a.n4;
        const float4 m0 = init ? a.M0[jm] : make_float4(0.f, 0.f, 0.f, 0.f);

        // ---- stage 1: sort each half, keep the first K ----
        uint64_t k1[E], k2[E];
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            if (e < S) {
                const uint32_t inv = ~(uint32_t)e;
                k1[r] = ((uint64_t)f2ord(load_elem(x, a.bf16, base + e)) << 32) | inv;
                k2[r] = ((uint64_t)f2ord(load_elem(x, a.bf16, base + S + e)) << 32) | inv;
            } else {
                k1[r] = 0;  // below every finite score
                k2[r] = 0;
            }
        }
        sort_halves_desc<E>(k1, k2, lane);
        if (init) {  // the piece of M0 has arrived during the sort
            if (a.init_bf16) {
                const uint2 u = make_uint2(bf16_bits(m0.x) | (bf16_bits(m0.y) << 16),
                                           bf16_bits(m0.z) | (bf16_bits(m0.w) << 16));
                for (int b = 0; b < a.Bseq; b++) reinterpret_cast<uint2 *>(a.M)[b * a.n4 + jm] = u;
            } else {
                for (int b = 0; b < a.Bseq; b++) reinterpret_cast<float4 *>(a.M)[b * a.n4 + jm] = m0;
            }
        }
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            if (e < K) {
                sv[wv][0][e] = ord2f((uint32_t)(k1[r] >> 32));
                si[wv][0][e] = ~(uint32_t)k1[r];
                sv[wv][1][e] = ord2f((uint32_t)(k2[r] >> 32));
                si[wv][1][e] = ~(uint32_t)k2[r];
            }
        }
        wave_sync();

        // ---- stage 2: exact sums of the pruned rank pairs ----
        uint64_t ck[E2];
        uint32_t cn[E2];
#pragma unroll
        for (int r = 0; r < E2; r++) {
            ck[r] = 0;  // empty: after every real candidate
            cn[r] = 0xFFFFFFFFu;
            const uint32_t ab = tabv[r];
            if (ab != kNoPair) {
                const int ra = (int)(ab >> 8), rb = (int)(ab & 0xFF);
                float hi, lo;
                two_sum(sv[wv][0][ra], sv[wv][1][rb], hi, lo);
                ck[r] = ((uint64_t)f2ord(hi) << 32) | f2ord(lo);
                cn[r] = si[wv][0][ra] * (uint32_t)S + si[wv][1][rb];
            }
        }
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
            uint32_t *xh = reinterpret_cast<uint32_t *>(sv[wv][0]);
            uint32_t *xl = reinterpret_cast<uint32_t *>(sv[wv][1]);
            uint32_t *xn = si[wv][0];
            // 64 survivors at a time (more than 64 is rare)
            for (int base = 0; base < tot; base += 64) {
                wave_sync();  // earlier reads of sv/si are done
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
        wave_sync();  // sv/si are rewritten by the next item

        // ---- weights: softmax over the K selected scores ----
        const uint64_t key = ck[0];
        const uint32_t n = cn[0];
        const float hi = ord2f((uint32_t)(key >> 32));
        const float lo = ord2f((uint32_t)key);
        const float hi0 = __shfl(hi, 0, 64);
        const float lo0 = __shfl(lo, 0, 64);
        const float ex = lane < K ? expf((hi - hi0) + (lo - lo0)) : 0.0f;
        float z = ex;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
        const float w = ex / z;

        if (a.hist != nullptr) {
            // write-slot utilisation: one count per selected slot of head h
            if (lane < K) atomicAdd(&a.hist[(int64_t)(ht % H32) * a.sqrtN * a.sqrtN + n], 1u);
        } else if (a.rec == nullptr) {
            if (lane < K) {
                const int64_t o = (int64_t)ht * K + lane;
                if (list == 0) {
                    a.Iw[o] = (int32_t)n;
                    a.kw[o] = w;
                } else {
                    a.Ir[o] = (int32_t)n;
                    a.qw[o] = w;
                }
            }
        } else {
            // record of chain (b, h) at token t; ht = (b*T + t)*H + h
            const uint32_t bt = ht / H32;
            const uint32_t h = ht - bt * H32;
            const uint32_t b = bt / T32;
            const uint32_t t = bt - b * T32;
            uint32_t *rec = a.rec + (((int64_t)(b * H32 + h) * T32) + t) * a.rec_dwords;
            if (list == 0) {
                if (lane < a.Wp) {
                    const bool ok = lane < K;
                    const float c = be * w;
                    rec[lane] = ok ? n : 0u;
                    reinterpret_cast<float *>(rec)[a.Wp + lane] = ok ? al * (1.0f - c) : 1.0f;
                    reinterpret_cast<float *>(rec)[2 * a.Wp + lane] = ok ? c : 0.0f;
                    reinterpret_cast<float *>(rec)[3 * a.Wp + 2 * a.Rp + lane] = ok ? w : 0.0f;
                }
            } else {
                if (lane < a.Rp) {
                    const bool ok = lane < K;
                    rec[3 * a.Wp + lane] = ok ? n : 0u;
                    reinterpret_cast<float *>(rec)[3 * a.Wp + a.Rp + lane] = ok ? w : 0.0f;
                }
            }
        }
    }
}

template <int E>
__global__ __launch_bounds__(256) void select_kernel(SelArgs a)
{
    select_body<E, false>(a);
}

// The variant that also copies M0 is held to the occupancy of the plain one
// (five wavefronts per SIMD), which its extra registers would otherwise lower;
// it fits without spilling up to sqrtN = 128 (E <= 2).
template <int E>
__global__ __launch_bounds__(256, 5) void select_init_kernel(SelArgs a)
{
    select_body<E, true>(a);
}

// The candidate columns of every list length K, built once per process (a
// thread-safe static) rather than on every launch.
struct HookTable {
    uint16_t pair[kTabMax];
    int rest;
};

const HookTable &hook_table(int K)
{
    static const std::array<HookTable, kMaxK + 1> tables = [] {
        std::array<HookTable, kMaxK + 1> t{};
        for (int k = 1; k <= kMaxK; k++) {
            for (int i = 0; i < kTabMax; i++) t[k].pair[i] = hook_pair(k, i / 64, i % 64);
            t[k].rest = hook_rest(k);
        }
        return t;
    }();
    return tables[K];
}

template <int E>
hipError_t launch_e(const SelArgs &args, hipStream_t st)
{
    const int64_t items = args.lists * args.n_ht;
    int64_t blocks = (items + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    // the copy of M0 is a separate instantiation: its registers would lower
    // the occupancy of every other selection
    if constexpr (E <= 2) {
        if (args.M0) {
            hipLaunchKernelGGL(select_init_kernel<E>, dim3((unsigned)blocks), dim3(256), 0, st,
                               args);
            return hipGetLastError();
        }
    } else if (args.M0) {
        return hipErrorInvalidValue;  // select_can_init rules this out
    }
    hipLaunchKernelGGL(select_kernel<E>, dim3((unsigned)blocks), dim3(256), 0, st, args);
    return hipGetLastError();
}

}  // namespace

// Item i of a full selection (both lists, all tokens) copies float4s
// [64 i, 64 i + 64) of M0: the items must cover the n/4 float4s of a slab.
// Only up to sqrtN = 128: wider instantiations cannot hold the copy's
// registers at the same occupancy (at sqrtN = 512 the selection took 24.1 ms
// instead of 23.1 + 0.4 for the separate copy).
bool select_can_init(const Shape &s)
{
    const int64_t n = (int64_t)s.H * s.N() * s.d_v;
    return s.sqrtN <= 128 && n % 4 == 0 && 2 * s.ht() * 64 >= n / 4;
}

hipError_t launch_select(const Shape &s, const void *kp, const void *qp, bool bf16,
                         int32_t *Iw, float *kw, int32_t *Ir, float *qw, uint32_t *rec,
                         const float *alpha, const float *beta, hipStream_t st, uint32_t *hist,
                         int64_t t0, int64_t tn, const SelInit *init)
{
    if (tn < 0) tn = s.T - t0;
    SelArgs a{};
    a.kp = kp;
    a.qp = qp;
    a.bf16 = bf16 ? 1 : 0;
    a.T = s.T;
    a.H = s.H;
    a.sqrtN = s.sqrtN;
    a.W = s.W;
    a.R = s.R;
    a.t0 = t0;
    a.tn = tn;
    a.n_ht = (int64_t)s.B * tn * s.H;
    a.Iw = Iw;
    a.kw = kw;
    a.Ir = Ir;
    a.qw = qw;
    a.rec = rec;
    const RecLayout L(s.W, s.R);
    a.rec_dwords = L.dwords();
    a.Wp = L.Wp;
    a.Rp = L.Rp;
    a.alpha = alpha;
    a.beta = beta;
    a.hist = hist;
    a.lists = hist ? 1 : 2;
    if (init) {
        // only for a full selection whose items cover M0 (select_can_init)
        if (hist || tn != s.T || !select_can_init(s)) return hipErrorInvalidValue;
        a.M0 = reinterpret_cast<const float4 *>(init->M0);
        a.M = init->M;
        a.n4 = (int64_t)s.H * s.N() * s.d_v / 4;
        a.Bseq = s.B;
        a.init_bf16 = init->state_bf16 ? 1 : 0;
    }
    for (int list = 0; list < 2; list++) {
        const HookTable &t = hook_table(list ? s.R : s.W);
        memcpy(a.tab[list], t.pair, sizeof t.pair);
        a.tabn[list] = t.rest;
    }
    if (s.sqrtN <= 64) return launch_e<1>(a, st);
    if (s.sqrtN <= 128) return launch_e<2>(a, st);
    if (s.sqrtN <= 256) return launch_e<4>(a, st);
    if (s.sqrtN <= 512) return launch_e<8>(a, st);
    return launch_e<16>(a, st);
}

}  // namespace sdm
