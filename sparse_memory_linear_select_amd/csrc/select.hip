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
#include "select_device.h"

#include <array>
#include <cstring>

namespace sdm {
namespace {

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
        uint64_t kk[2][E];
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            if (e < S) {
                const uint32_t inv = ~(uint32_t)e;
                kk[0][r] = ((uint64_t)f2ord(load_elem(x, a.bf16, base + e)) << 32) | inv;
                kk[1][r] = ((uint64_t)f2ord(load_elem(x, a.bf16, base + S + e)) << 32) | inv;
            } else {
                kk[0][r] = 0;  // below every finite score
                kk[1][r] = 0;
            }
        }
        sort_desc<2, E>(kk, lane);
        if (init) {  // the piece of M0 has arrived during the sort
            if (a.init_bf16) {
                const uint2 u = make_uint2(bf16_pack2(m0.x, m0.y), bf16_pack2(m0.z, m0.w));
                for (int b = 0; b < a.Bseq; b++) reinterpret_cast<uint2 *>(a.M)[b * a.n4 + jm] = u;
            } else {
                for (int b = 0; b < a.Bseq; b++) reinterpret_cast<float4 *>(a.M)[b * a.n4 + jm] = m0;
            }
        }
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            if (e < K) {
                sv[wv][0][e] = ord2f((uint32_t)(kk[0][r] >> 32));
                si[wv][0][e] = ~(uint32_t)kk[0][r];
                sv[wv][1][e] = ord2f((uint32_t)(kk[1][r] >> 32));
                si[wv][1][e] = ~(uint32_t)kk[1][r];
            }
        }
        wave_sync();

        // ---- stage 2: exact sums of the pruned rank pairs ----
        uint64_t key;
        uint32_t n;
        select_pairs<E2>(sv[wv][0], sv[wv][1], si[wv][0], si[wv][1], tabv, K, rest, S, lane, key, n);
        wave_sync();  // sv/si are rewritten by the next item

        // ---- weights: softmax over the K selected scores ----
        const float w = select_weight(key, K, lane);

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

}  // namespace

const uint16_t *hook_columns(int K, int *rest)
{
    const HookTable &t = hook_table(K);
    *rest = t.rest;
    return t.pair;
}

namespace {

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
