// One-token step (decode): the W writes of token t, then its R reads, which
// see those writes (the write of the explainer "Sparse Delta Memory：通过稀疏性
// 扩展线性 RNN 的状态容量", §3.1 step 2, then the read of step 3).  With one
// token there is nothing to schedule across time, so a single kernel does
// both: one wavefront per (chain, 128-byte row slice) gathers, updates and
// stores the written rows, then gathers the read rows (a read of a slot written by the same
// token finds the new row) and sums them into y.  Only the wavefront that
// wrote a row slice reads it back, so no other ordering is needed.
#include "select_device.h"
#include "tp_device.h"

#include <atomic>

namespace sdm {

// Compute units of the current device (looked up once per device; threads
// that race here store the same value).
int compute_units()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

struct DecArgs {
    const uint32_t *rec;  // records [chain] (one token)
    const void *v;        // [B][1][H][d_v]
    float *y;             // [B][1][H][d_v]
    void *M;              // [chain][N][d_v] float32, bfloat16 or E4M3
    float ssc, sisc;      // E4M3 state: 2^s, 2^-s
    int64_t N;
    int H, d_v, W, R, Wp, Rp, rec_dwords;
    int64_t chains;
};

// Lanes per row slice: 128 bytes for a float32 or bfloat16 state (8 or 16
// lanes: for one token, more and smaller slices spread the gathers over more
// compute units); 16 lanes (64 bytes) for an E4M3 state, so that a wave
// keeps 4 row groups and at most 16 references per group in registers.
template <int ST>
constexpr int dec_lpr()
{
    return ST == kStateF32 ? 8 : 16;
}

template <bool BF16, int ST, int NK>
__global__ __launch_bounds__(64) void rw_decode_kernel(DecArgs a, int nslice)
{
    using S = StateRow<ST>;
    const S st(a.ssc, a.sisc);
    constexpr int kLPR = dec_lpr<ST>(), kRPI = 64 / kLPR;
    const int lane = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int slice = (int)(unit % nslice);
    const int64_t chain = unit / nslice;
    const int g = lane / kLPR, q = lane % kLPR;
    const int col = slice * 4 * kLPR + q * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;
    const int64_t vy = chain * a.d_v + colc;  // [B][1][H][d_v]: chain = b*H + h
    const rsrc_t Mr = make_rsrc(static_cast<char *>(a.M) + chain * a.N * a.d_v * S::kElem,
                                (uint32_t)(a.N * a.d_v * S::kElem));
    const uint32_t rowb = (uint32_t)a.d_v * S::kElem;
    const uint32_t *rc = a.rec + chain * a.rec_dwords;
    const float *rf = reinterpret_cast<const float *>(rc);

    // this lane's record words, all loaded before the first store (the
    // stores go through a buffer descriptor the compiler cannot tell apart
    // from the records): row group g takes writes and reads g, g + kRPI, ...
    uint32_t wslot[NK], rslot[NK];
    float wa[NK], wc[NK], rq[NK];
#pragma unroll
    for (int i = 0; i < NK; i++) {  // unconditional loads (indices clamped into the record)
        const int w = g + i * kRPI < a.W ? g + i * kRPI : 0;
        const int r = g + i * kRPI < a.R ? g + i * kRPI : 0;
        wslot[i] = rc[w];
        wa[i] = rf[a.Wp + w];
        wc[i] = rf[2 * a.Wp + w];
        rslot[i] = rc[3 * a.Wp + r];
        rq[i] = rf[3 * a.Wp + a.Rp + r];
    }
#pragma unroll
    for (int i = 0; i < NK; i++) {
        const int k = g + i * kRPI;
        wslot[i] = (col_ok & (k < a.W)) ? (wslot[i] & kSlotMask) * rowb + col * S::kElem : kOff;
        rslot[i] = (col_ok & (k < a.R)) ? (rslot[i] & kSlotMask) * rowb + col * S::kElem : kOff;
        rq[i] = k < a.R ? rq[i] : 0.f;  // out-of-range rows load zero anyway
    }
    const float4 vv = load_v<BF16>(a.v, vy);

    // writes (rows are distinct within a token)
    typename S::Raw old[NK];
#pragma unroll
    for (int i = 0; i < NK; i++) old[i] = st.load_raw(Mr, wslot[i]);
#pragma unroll
    for (int i = 0; i < NK; i++) st.store(st.round(fma4(wa[i], st.widen(old[i]), wc[i], vv)), Mr, wslot[i]);
    // the reads below are ordered after the stores at workgroup scope: the
    // workgroup is this one wavefront, whose vector memory operations all go
    // through one CU's L1 (no L2 write-back or invalidation is needed)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    // reads of the updated state
    typename S::Raw row[NK];
#pragma unroll
    for (int i = 0; i < NK; i++) row[i] = st.load_raw(Mr, rslot[i]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NK; i++) {
        const float4 x = st.widen(row[i]);
        acc.x = fmaf(rq[i], x.x, acc.x);
        acc.y = fmaf(rq[i], x.y, acc.y);
        acc.z = fmaf(rq[i], x.z, acc.z);
        acc.w = fmaf(rq[i], x.w, acc.w);
    }
#pragma unroll
    for (int m = kLPR; m < 64; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m, 64);
        acc.y += __shfl_xor(acc.y, m, 64);
        acc.z += __shfl_xor(acc.z, m, 64);
        acc.w += __shfl_xor(acc.w, m, 64);
    }
    if (g == 0 && col_ok) *reinterpret_cast<float4 *>(a.y + chain * a.d_v + col) = acc;
}

template <int ST>
hipError_t launch_state(const Shape &s, const DecArgs &a, bool bf16, hipStream_t st)
{
    constexpr int kLPR = dec_lpr<ST>(), kRPI = 64 / kLPR;
    const int nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    // one wavefront per workgroup: few units, spread over as many CUs as possible
    const dim3 grid((unsigned)(a.chains * nslice));
    const int K = s.W > s.R ? s.W : s.R;
    const int nk = (K + kRPI - 1) / kRPI;
#define SDM_DEC(NK_)                                                                              \
    if (nk <= NK_) {                                                                              \
        if (bf16) hipLaunchKernelGGL((rw_decode_kernel<true, ST, NK_>), grid, dim3(64), 0, st, a, \
                                     nslice);                                                     \
        else hipLaunchKernelGGL((rw_decode_kernel<false, ST, NK_>), grid, dim3(64), 0, st, a,     \
                                nslice);                                                          \
        return hipGetLastError();                                                                 \
    }
    SDM_DEC(1) SDM_DEC(2) SDM_DEC(4) SDM_DEC(8) SDM_DEC(16)
#undef SDM_DEC
    return hipErrorInvalidValue;
}

// The whole step in one launch.  A workgroup of four wavefronts serves one
// chain (b, h) and a range of its row slices.  It first selects the chain's
// slots itself, with the selection kernel's steps (so the same slots and
// weights): wavefront (list, half) sorts one half of k' (list 0) or q'
// (list 1); of each list's two wavefronts one merges the pairs of hooks 0
// and 1 while the other sorts those of hooks >= 2, and the first merges the
// two and takes the softmax; the write coefficients a = alpha(1 - beta k),
// c = beta k go to LDS with the slots.  Then 1, 2 or 4 of the wavefronts
// (as many as keep about one workgroup per compute unit) take a row slice
// each, as the two-launch kernel does, but gather the written and the read
// rows at once; while the gathers are in flight every wavefront looks
// for reads whose slot the token also writes, and such a read takes the new
// row from the LDS copy of the rows its wavefront just wrote (the stored
// values), so no gather waits on the stores.  Every workgroup of a chain
// repeats the selection: for one token the chip has far more compute units
// than lists, and the repeat costs no time, while records in memory and a
// second launch would.
struct DecFArgs {
    const void *kp, *qp, *v;
    const float *alpha, *beta;
    float *y;
    void *M;
    float ssc, sisc;  // E4M3 state: 2^s, 2^-s
    int64_t N;
    int sqrtN, d_v, W, R, bf16;
    int nslice, groups;  // row slices per chain; workgroups per chain
    int rw, spw;         // wavefronts per workgroup that take row slices (1, 2 or 4); slices each
    uint16_t tab[2][kTabMax];
    int tabn[2];
};

template <int E, int ST>
__global__ __launch_bounds__(256) void rw_decode_fused_kernel(DecFArgs a)
{
    using S = StateRow<ST>;
    using Raw = typename S::Raw;
    const S st(a.ssc, a.sisc);
    constexpr int kLPR = dec_lpr<ST>(), kRPI = 64 / kLPR, NK = kMaxK / kRPI;
    __shared__ float sv[2][2][64];
    __shared__ uint32_t si[2][2][64];
    __shared__ uint32_t yh[2][64], yl[2][64], yn[2][64];  // sorted pairs of hooks >= 2
    __shared__ __align__(16) uint32_t wsl_s[kMaxK];
    __shared__ uint32_t rsl_s[kMaxK];
    __shared__ float wa_s[kMaxK], wc_s[kMaxK], rq_s[kMaxK];
    __shared__ int rmatch_s[kMaxK];
    __shared__ Raw wrow[4][kMaxK][kLPR];  // rows each row wavefront wrote, as stored
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int list = wv >> 1, half = wv & 1;
    // one token: the chain b*H + h is also the head-token's index
    const uint32_t chain = blockIdx.x / (uint32_t)a.groups;
    const int grp = (int)(blockIdx.x - chain * (uint32_t)a.groups);
    const int Sq = a.sqrtN;
    const int K = list ? a.R : a.W;
    const int rest = a.tabn[list];

    float al = 0.0f, be = 0.0f;
    if (wv == 0) {
        al = a.alpha[chain];
        be = a.beta[chain];
    }
    // this wavefront's candidate columns: 0-2 (half 0) or 3, 4 (half 1)
    uint16_t tabv[3];
#pragma unroll
    for (int r = 0; r < 3; r++) {
        const int c = half ? 3 + r : r;
        tabv[r] = c < 5 ? a.tab[list][c * 64 + lane] : kNoPair;
    }

    // ---- selection, stage 1: this wavefront's half, sorted; first K kept ----
    {
        const void *x = list ? a.qp : a.kp;
        const int64_t base = (int64_t)chain * 2 * Sq + half * Sq;
        uint64_t kk[1][E];
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            kk[0][r] = e < Sq ? ((uint64_t)f2ord(load_elem(x, a.bf16, base + e)) << 32) |
                                    ~(uint32_t)e
                              : 0;  // below every finite score
        }
        sort_desc<1, E>(kk, lane);
#pragma unroll
        for (int r = 0; r < E; r++) {
            const int e = lane * E + r;
            if (e < K) {
                sv[list][half][e] = ord2f((uint32_t)(kk[0][r] >> 32));
                si[list][half][e] = ~(uint32_t)kk[0][r];
            }
        }
    }
    __syncthreads();

    // ---- stage 2 (see select_pairs: the same candidates, split over the
    // list's two wavefronts; every candidate is kept until the last merge) ----
    uint64_t key = 0;
    uint32_t n = 0xFFFFFFFFu;
    {
        const float *v1 = sv[list][0], *v2 = sv[list][1];
        const uint32_t *i1 = si[list][0], *i2 = si[list][1];
        if (half == 0) {
            // hook 0: columns 0 and 1 arrive sorted; hook 1: column 2 bitonic
            uint64_t ck[3];
            uint32_t cn[3];
#pragma unroll
            for (int r = 0; r < 3; r++) pair_entry(v1, v2, i1, i2, tabv[r], Sq, ck[r], cn[r]);
            if (K >= 2) col_merge(ck[0], cn[0], ck[1], cn[1], lane);
            if (K >= 4) {
                col_bitonic(ck[2], cn[2], lane);
                col_merge(ck[0], cn[0], ck[2], cn[2], lane);
            }
            key = ck[0];
            n = cn[0];
        } else if (rest > 0) {
            // hooks >= 2: columns 3 and 4, unsorted
            uint64_t ck[2];
            uint32_t cn[2];
#pragma unroll
            for (int r = 0; r < 2; r++) pair_entry(v1, v2, i1, i2, tabv[r], Sq, ck[r], cn[r]);
            col_sort(ck[0], cn[0], lane);
            if (rest > 64) {
                col_sort(ck[1], cn[1], lane);
                col_merge(ck[0], cn[0], ck[1], cn[1], lane);
            }
            yh[list][lane] = (uint32_t)(ck[0] >> 32);
            yl[list][lane] = (uint32_t)ck[0];
            yn[list][lane] = cn[0];
        }
    }
    __syncthreads();
    if (half == 0) {
        if (rest > 0) {
            const int r = 63 - lane;
            col_merge_rev(key, n, ((uint64_t)yh[list][r] << 32) | yl[list][r], yn[list][r], lane);
        }
        const float w = select_weight(key, K, lane);
        if (lane < K) {
            if (list == 0) {
                const float c = be * w;
                wsl_s[lane] = n;
                wa_s[lane] = al * (1.0f - c);
                wc_s[lane] = c;
            } else {
                rsl_s[lane] = n;
                rq_s[lane] = w;
            }
        }
    }
    __syncthreads();

    // ---- writes and reads: wavefronts 0 .. rw-1 take row slices ----
    const int g = lane / kLPR, q = lane % kLPR;
    const rsrc_t Mr = make_rsrc(static_cast<char *>(a.M) + (int64_t)chain * a.N * a.d_v * S::kElem,
                                (uint32_t)(a.N * a.d_v * S::kElem));
    const uint32_t rowb = (uint32_t)a.d_v * S::kElem;
    // row group g takes writes and reads g, g + kRPI, ...
    uint32_t wsl[NK], rsl[NK];
    float wa[NK], wc[NK], rq[NK];
    // (entries past W or R hold stale LDS: their gathers and stores are masked,
    // and a read weight past R is zeroed)
#pragma unroll
    for (int i = 0; i < NK; i++) {
        const int k = g + i * kRPI;
        wsl[i] = wsl_s[k];
        wa[i] = wa_s[k];
        wc[i] = wc_s[k];
        rsl[i] = rsl_s[k];
        const float w = rq_s[k];
        rq[i] = k < a.R ? w : 0.0f;
    }
    // gathers of one slice: the written rows and every read row
    Raw old[NK], row[NK];
    float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
    int slice = grp * a.spw * a.rw + wv;
    bool have = wv < a.rw && slice < a.nslice;
    auto gather = [&](int sl) {
        const int col = sl * 4 * kLPR + q * 4;
        const bool col_ok = col < a.d_v;
        const int64_t vy = (int64_t)chain * a.d_v + (col_ok ? col : 0);
        vv = a.bf16 ? load_v<true>(a.v, vy) : load_v<false>(a.v, vy);
#pragma unroll
        for (int i = 0; i < NK; i++) {
            const int k = g + i * kRPI;
            old[i] = st.load_raw(Mr, (col_ok & (k < a.W)) ? wsl[i] * rowb + col * S::kElem : kOff);
        }
#pragma unroll
        for (int i = 0; i < NK; i++) {
            const int k = g + i * kRPI;
            row[i] = st.load_raw(Mr, (col_ok & (k < a.R)) ? rsl[i] * rowb + col * S::kElem : kOff);
        }
    };
    if (have) gather(slice);

    // ---- meanwhile: the write of each read's slot by this token, if any
    // (slots within a list are distinct); four lanes per read, 16 writes each ----
    {
        const int i = wv * 16 + (lane >> 2);
        const int j0 = (lane & 3) * 16;
        int m = -1;
        if (i < a.R) {
            const uint32_t sl = rsl_s[i];
            const uint4 *w4 = reinterpret_cast<const uint4 *>(wsl_s + j0);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint4 ws = w4[u];
                const int j = j0 + 4 * u;
                if (j < a.W && ws.x == sl) m = j;
                if (j + 1 < a.W && ws.y == sl) m = j + 1;
                if (j + 2 < a.W && ws.z == sl) m = j + 2;
                if (j + 3 < a.W && ws.w == sl) m = j + 3;
            }
        }
        m = max(m, __shfl_xor(m, 1, 64));
        m = max(m, __shfl_xor(m, 2, 64));
        if ((lane & 3) == 0 && i < a.R) rmatch_s[i] = m;
    }
    __syncthreads();
    if (wv >= a.rw) return;
    int rm[NK];
#pragma unroll
    for (int i = 0; i < NK; i++) {
        const int k = g + i * kRPI;
        rm[i] = k < a.R ? rmatch_s[k] : -1;
    }

    for (int u = 0; have;) {
        const int col = slice * 4 * kLPR + q * 4;
        const bool col_ok = col < a.d_v;
        wave_sync();  // the previous slice's reads of wrow are done
#pragma unroll
        for (int i = 0; i < NK; i++) {
            const int k = g + i * kRPI;
            const float4 nw = st.round(fma4(wa[i], st.widen(old[i]), wc[i], vv));
            st.store(nw, Mr, (col_ok & (k < a.W)) ? wsl[i] * rowb + col * S::kElem : kOff);
            if (k < a.W) wrow[wv][k][q] = st.pack(nw);
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < NK; i++)
            if (rm[i] >= 0) row[i] = wrow[wv][rm[i]][q];
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < NK; i++) {
            const float4 x = st.widen(row[i]);
            acc.x = fmaf(rq[i], x.x, acc.x);
            acc.y = fmaf(rq[i], x.y, acc.y);
            acc.z = fmaf(rq[i], x.z, acc.z);
            acc.w = fmaf(rq[i], x.w, acc.w);
        }
#pragma unroll
        for (int m = kLPR; m < 64; m <<= 1) {
            acc.x = xor_add(acc.x, m);
            acc.y = xor_add(acc.y, m);
            acc.z = xor_add(acc.z, m);
            acc.w = xor_add(acc.w, m);
        }
        if (g == 0 && col_ok)
            *reinterpret_cast<float4 *>(a.y + (int64_t)chain * a.d_v + col) = acc;
        if (++u >= a.spw) break;
        slice = (grp * a.spw + u) * a.rw + wv;
        have = slice < a.nslice;
        if (have) gather(slice);
    }
}


template <int ST>
hipError_t launch_fused_state(const Shape &s, DecFArgs &a, hipStream_t st)
{
    constexpr int kLPR = dec_lpr<ST>();
    a.nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    const int64_t chains = (int64_t)s.B * s.H;
    // Every workgroup repeats its chain's selection, so a compute unit that
    // holds two of them takes twice as long over it: about one workgroup per
    // compute unit, with 1, 2 or 4 of its wavefronts taking row slices (more
    // workgroups per chain spread the gathers over more compute units), and
    // more slices per wavefront only beyond that.
    const int cus = compute_units();
    const int64_t per = (int64_t)cus;
    a.rw = chains * a.nslice <= per ? 1 : (chains * ((a.nslice + 1) / 2) <= per ? 2 : 4);
    int spw = 1;
    while (chains * ((a.nslice + a.rw * spw - 1) / (a.rw * spw)) > per && a.rw * spw < a.nslice)
        spw *= 2;
    a.spw = spw;
    a.groups = (a.nslice + a.rw * spw - 1) / (a.rw * spw);
    const int64_t blocks = chains * a.groups;
    if (blocks >= (int64_t)1 << 31) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
#define SDM_DECF(E_)                                                                            case E_:                                                                                        hipLaunchKernelGGL((rw_decode_fused_kernel<E_, ST>), grid, dim3(256), 0, st, a);           return hipGetLastError();
    switch ((s.sqrtN + 63) / 64) {
        SDM_DECF(1)
        SDM_DECF(2)
    case 3:
        SDM_DECF(4)
    case 5:
    case 6:
    case 7:
        SDM_DECF(8)
    default: return hipErrorInvalidValue;
    }
#undef SDM_DECF
}

}  // namespace

bool decode_fused_supported(const Shape &s)
{
    return decode_supported(s) && s.sqrtN <= 512;
}

hipError_t launch_decode_fused(const Shape &s, const void *kp, const void *qp, const void *v,
                               bool bf16, const float *alpha, const float *beta, float *y,
                               void *M, StateFmt fmt, hipStream_t st)
{
    if (!decode_fused_supported(s)) return hipErrorInvalidValue;
    DecFArgs a{};
    a.kp = kp;
    a.qp = qp;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.y = y;
    a.M = M;
    a.ssc = ldexpf(1.0f, fmt.scale_log2);
    a.sisc = ldexpf(1.0f, -fmt.scale_log2);
    a.N = s.N();
    a.sqrtN = s.sqrtN;
    a.d_v = s.d_v;
    a.W = s.W;
    a.R = s.R;
    a.bf16 = bf16 ? 1 : 0;
    for (int list = 0; list < 2; list++) {
        const uint16_t *t = hook_columns(list ? s.R : s.W, &a.tabn[list]);
        for (int i = 0; i < kTabMax; i++) a.tab[list][i] = t[i];
    }
    switch (fmt.type) {
        case kStateBF16: return launch_fused_state<kStateBF16>(s, a, st);
        case kStateFP8: return launch_fused_state<kStateFP8>(s, a, st);
        default: return launch_fused_state<kStateF32>(s, a, st);
    }
}

bool decode_supported(const Shape &s)
{
    return s.T == 1 && s.d_v % 4 == 0 && (double)s.N() * s.d_v * 4.0 <= 2147483648.0;
}

hipError_t launch_rw_decode(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, void *M, StateFmt fmt, hipStream_t st)
{
    DecArgs a{};
    const RecLayout L(s.W, s.R);
    a.rec = rec;
    a.v = v;
    a.y = y;
    a.M = M;
    a.N = s.N();
    a.H = s.H;
    a.d_v = s.d_v;
    a.W = s.W;
    a.R = s.R;
    a.Wp = L.Wp;
    a.Rp = L.Rp;
    a.rec_dwords = L.dwords();
    a.chains = (int64_t)s.B * s.H;
    a.ssc = ldexpf(1.0f, fmt.scale_log2);
    a.sisc = ldexpf(1.0f, -fmt.scale_log2);
    switch (fmt.type) {
        case kStateBF16: return launch_state<kStateBF16>(s, a, bf16, st);
        case kStateFP8: return launch_state<kStateFP8>(s, a, bf16, st);
        default: return launch_state<kStateF32>(s, a, bf16, st);
    }
}

}  // namespace sdm
