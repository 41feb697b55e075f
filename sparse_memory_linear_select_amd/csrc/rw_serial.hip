// Token-serial gated delta write + sparse read (the recurrence of the SDM core).
//
// For every token t of a chain (sequence b, head h), in order:
//   write  for each selected slot i: M[i] <- a_i * M[i] + c_i * v_t with
//          a_i = alpha_t (1 - beta_t k^(i)) and c_i = beta_t k^(i), which is
//          the forget gate followed by the delta write of the explainer "Sparse
//          Delta Memory：通过稀疏性扩展线性 RNN 的状态容量", §3.1 step 2 (and
//          "Technical Summary: Sparse Delta Memory (SDM)", Core Mechanism 3)
//          written as one affine map; other rows are not touched;
//   read   y_t = sum_i q^(i) M[i] over the read set, after the write (§3.1
//          step 3; Core Mechanism 4).
// Columns of M never interact, so the work splits into independent units
// (chain, 16-column slice), one 64-lane wavefront each: 4 lanes x float4 cover
// the 16 columns of one row and the 16 row groups of the wave take 16 slot
// references at a time.  The rows of token t+P are gathered while token t is
// processed; a prefetched row that one of the previous P-1 tokens wrote (or,
// for a read, the same token) is taken from the wave's LDS copy of those
// writes instead, as recorded in the slot word by the planner.
//
// rw_simple_kernel is the plain version (one column per lane, no prefetch),
// used when d_v is not a multiple of 4.
#include "sdm_internal.h"

#ifndef SDM_RW_DEPTH
#define SDM_RW_DEPTH 2
#endif

namespace sdm {
namespace {

constexpr int kDepth = SDM_RW_DEPTH;  // cross-token prefetch depth

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int K, typename T>
__device__ __forceinline__ void load_k(const T *p, T (&out)[K])
{
    if constexpr (K == 4 && sizeof(T) == 4) {
        const uint4 x = *reinterpret_cast<const uint4 *>(p);
        out[0] = __builtin_bit_cast(T, x.x);
        out[1] = __builtin_bit_cast(T, x.y);
        out[2] = __builtin_bit_cast(T, x.z);
        out[3] = __builtin_bit_cast(T, x.w);
    } else if constexpr (K == 8 && sizeof(T) == 4) {
        const uint4 x = *reinterpret_cast<const uint4 *>(p);
        const uint4 z = *reinterpret_cast<const uint4 *>(p + 4);
        out[0] = __builtin_bit_cast(T, x.x);
        out[1] = __builtin_bit_cast(T, x.y);
        out[2] = __builtin_bit_cast(T, x.z);
        out[3] = __builtin_bit_cast(T, x.w);
        out[4] = __builtin_bit_cast(T, z.x);
        out[5] = __builtin_bit_cast(T, z.y);
        out[6] = __builtin_bit_cast(T, z.z);
        out[7] = __builtin_bit_cast(T, z.w);
    } else if constexpr (K == 2 && sizeof(T) == 4) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        out[0] = __builtin_bit_cast(T, x.x);
        out[1] = __builtin_bit_cast(T, x.y);
    } else {
#pragma unroll
        for (int i = 0; i < K; i++) out[i] = p[i];
    }
}

template <bool BF16>
__device__ __forceinline__ float4 load_v4(const void *v, int64_t off)
{
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(v) + off);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
        return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(v) + off);
    }
}

struct RWArgs {
    const uint32_t *rec;
    const void *v;
    float *y, *M;
    int64_t T, N;
    int H, d_v, W, R, Wp, Rp, rec_dwords;
    int64_t nslice, units, per_xcd;
};

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOff = 0x80000000u;  // out-of-range buffer offset: loads give 0, stores drop
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer descriptor flags

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ float4 buf_load4(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ void buf_store4(float4 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, (int)off, 0, 0);
}

__device__ __forceinline__ float4 fma4(float a, float4 x, float c, float4 v)
{
    return make_float4(fmaf(a, x.x, c * v.x), fmaf(a, x.y, c * v.y), fmaf(a, x.z, c * v.z),
                       fmaf(a, x.w, c * v.w));
}

// One wavefront = one unit (chain, slice of 4*LPR columns): LPR lanes x float4
// cover one row of the slice, 64/LPR row groups take that many references at
// a time (NW write and NR read references per group per token).  The steady
// state is branch-free: masked lanes use out-of-range buffer offsets, tokens
// past the end are clamped for loads and masked for stores, so the compiler
// can keep the P-token prefetch in flight across iterations.
template <int LPR, int NW, int NR, int P, bool BF16>
__global__ __launch_bounds__(256) void rw_serial_kernel(RWArgs a)
{
    __shared__ float4 ring[4][P][kMaxK][LPR];  // per wave: writes of the last P tokens
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    // the units of one chain sit on one XCD (workgroups are dealt round-robin)
    const int64_t lwg = (int64_t)(blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
    const int64_t unit = lwg * 4 + wv;
    if (unit >= a.units) return;
    const int64_t chain = unit / a.nslice;
    const int slice = (int)(unit - chain * a.nslice);
    const int g = lane / LPR;  // row group
    const int q = lane % LPR;  // float4 within the slice
    const int col = slice * 4 * LPR + q * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;  // clamped column for always-valid loads
    const int64_t b = chain / a.H;
    const int h = (int)(chain - b * a.H);
    const int64_t T = a.T;
    const uint32_t rowb = (uint32_t)a.d_v * 4u;
    const rsrc_t Mr = make_rsrc(a.M + chain * a.N * a.d_v, (uint32_t)(a.N * a.d_v * 4));
    const uint32_t *recc = a.rec + chain * T * a.rec_dwords;
    const int64_t hd = (int64_t)a.H * a.d_v;  // stride of one token in v and y
    const float *vf = reinterpret_cast<const float *>(a.v) + (b * T * a.H + h) * a.d_v + colc;
    const uint16_t *vh = reinterpret_cast<const uint16_t *>(a.v) + (b * T * a.H + h) * a.d_v + colc;
    float *ybase = a.y + (b * T * a.H + h) * a.d_v;
    bool okw[NW], okr[NR];
#pragma unroll
    for (int i = 0; i < NW; i++) okw[i] = col_ok & (g * NW + i < a.W);
#pragma unroll
    for (int i = 0; i < NR; i++) okr[i] = col_ok & (g * NR + i < a.R);

    uint32_t sw[2 * P][NW], sr[2 * P][NR];  // slot words, 2P tokens ahead
    float4 rw[P][NW], rr[P][NR];            // gathered rows, P tokens ahead
    float ma[P][NW], mc[P][NW], mq[P][NR];  // coefficients
    float4 mv[P];                           // v_t slice

    auto clampt = [&](int64_t t) { return t < 0 ? 0 : (t < T ? t : T - 1); };
    auto fwd = [](uint32_t s) {  // no short-circuit: keeps the code branch-free
        return ((s & kFwdValid) != 0) & (((s >> kFwdDShift) & kFwdDMask) < (uint32_t)P);
    };
    auto load_slots = [&](int64_t t, uint32_t (&ow)[NW], uint32_t (&orr)[NR]) {
        const uint32_t *r = recc + clampt(t) * a.rec_dwords;
        load_k<NW>(r + g * NW, ow);
        load_k<NR>(r + 3 * a.Wp + g * NR, orr);
    };
    auto load_rows = [&](int64_t t, const uint32_t (&iw)[NW], const uint32_t (&ir)[NR],
                         float4 (&ow)[NW], float4 (&orr)[NR], float (&oa)[NW], float (&oc)[NW],
                         float (&oq)[NR], float4 &ov) {
        const int64_t tc = clampt(t);
#pragma unroll
        for (int i = 0; i < NW; i++)
            ow[i] = buf_load4(Mr, (okw[i] & !fwd(iw[i])) ? (iw[i] & kSlotMask) * rowb + col * 4u : kOff);
#pragma unroll
        for (int i = 0; i < NR; i++)
            orr[i] = buf_load4(Mr, (okr[i] & !fwd(ir[i])) ? (ir[i] & kSlotMask) * rowb + col * 4u : kOff);
        if constexpr (BF16) {
            const uint2 u = *reinterpret_cast<const uint2 *>(vh + tc * hd);
            ov = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
        } else {
            ov = *reinterpret_cast<const float4 *>(vf + tc * hd);
        }
        const float *r = reinterpret_cast<const float *>(recc + tc * a.rec_dwords);
        load_k<NW>(r + a.Wp + g * NW, oa);
        load_k<NW>(r + 2 * a.Wp + g * NW, oc);
        load_k<NR>(r + 3 * a.Wp + a.Rp + g * NR, oq);
    };

    // The loop starts 2P tokens early: those trips only fill the prefetch
    // pipeline (their tokens are outside [0, T), so their stores are masked).
    // Issuing the first loads inside the loop, not in a separate prologue,
    // keeps the compiler's wait counts exact across the back-edge.
#pragma unroll
    for (int u = 0; u < 2 * P; u++) {
#pragma unroll
        for (int i = 0; i < NW; i++) sw[u][i] = 0;
#pragma unroll
        for (int i = 0; i < NR; i++) sr[u][i] = 0;
    }
#pragma unroll
    for (int u = 0; u < P; u++) {
        mv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < NW; i++) {
            rw[u][i] = mv[u];
            ma[u][i] = 0.f;
            mc[u][i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            rr[u][i] = mv[u];
            mq[u][i] = 0.f;
        }
    }

    for (int64_t t0 = -2 * P; t0 < T; t0 += 2 * P) {
        // y of this trip's tokens through a descriptor based at token t0 (only
        // offsets of tokens in [0, T) are ever used)
        const rsrc_t Yr = make_rsrc(ybase + t0 * hd, (uint32_t)(2 * P * hd * 4));
#pragma unroll
        for (int u = 0; u < 2 * P; u++) {
            const int pr = u % P;
            // ---- write: old row (prefetched, or forwarded from the LDS ring) ----
#pragma unroll
            for (int i = 0; i < NW; i++) {
                const uint32_t s = sw[u][i];
                const bool f = fwd(s);
                const int d = f ? (int)((s >> kFwdDShift) & kFwdDMask) : 0;
                const int wp = f ? (int)((s >> kFwdWShift) & kFwdWMask) : 0;
                const float4 fv = ring[wv][(pr - d + P) % P][wp][q];
                const float4 old = f ? fv : rw[pr][i];
                const float4 nv = fma4(ma[pr][i], old, mc[pr][i], mv[pr]);
                const bool live = (t0 + u >= 0) & (t0 + u < T);
                buf_store4(nv, Mr, (okw[i] & live) ? (s & kSlotMask) * rowb + col * 4u : kOff);
                ring[wv][pr][g * NW + i][q] = nv;
            }
            wave_sync();
            // ---- read of the post-write state ----
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < NR; i++) {
                const uint32_t s = sr[u][i];
                const bool f = fwd(s);
                const int d = f ? (int)((s >> kFwdDShift) & kFwdDMask) : 0;
                const int wp = f ? (int)((s >> kFwdWShift) & kFwdWMask) : 0;
                const float4 fv = ring[wv][(pr - d + P) % P][wp][q];
                const float4 val = f ? fv : rr[pr][i];
                const float qv = mq[pr][i];
                acc.x = fmaf(qv, val.x, acc.x);
                acc.y = fmaf(qv, val.y, acc.y);
                acc.z = fmaf(qv, val.z, acc.z);
                acc.w = fmaf(qv, val.w, acc.w);
            }
#pragma unroll
            for (int m = LPR; m < 64; m <<= 1) {
                acc.x += __shfl_xor(acc.x, m, 64);
                acc.y += __shfl_xor(acc.y, m, 64);
                acc.z += __shfl_xor(acc.z, m, 64);
                acc.w += __shfl_xor(acc.w, m, 64);
            }
            buf_store4(acc, Yr,
                       ((g == 0) & col_ok & (t0 + u >= 0) & (t0 + u < T)) ? (uint32_t)((u * hd + col) * 4) : kOff);
            wave_sync();
            // ---- prefetch: rows of token t+P, slot words of token t+2P ----
            load_rows(t0 + u + P, sw[(u + P) % (2 * P)], sr[(u + P) % (2 * P)], rw[pr], rr[pr],
                      ma[pr], mc[pr], mq[pr], mv[pr]);
            load_slots(t0 + u + 2 * P, sw[u], sr[u]);
            // keep each token's loads where they are issued: the scheduler
            // must not sink them into later tokens (that shortens the prefetch)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void rw_simple_kernel(RWArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= a.units) return;
    const int64_t chain = unit / a.nslice;
    const int slice = (int)(unit - chain * a.nslice);
    const int col = slice * 64 + lane;
    const bool ok = col < a.d_v;
    const int64_t b = chain / a.H;
    const int h = (int)(chain - b * a.H);
    float *Mc = a.M + chain * a.N * a.d_v + col;
    const uint32_t *recc = a.rec + chain * a.T * a.rec_dwords;
    for (int64_t t = 0; t < a.T; t++) {
        const uint32_t *r = recc + t * a.rec_dwords;
        const float *rf = reinterpret_cast<const float *>(r);
        const int64_t off = (((b * a.T + t) * a.H) + h) * a.d_v + col;
        float vt = 0.f;
        if (ok)
            vt = BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(a.v)[off] << 16)
                      : reinterpret_cast<const float *>(a.v)[off];
        for (int w = 0; w < a.W; w++) {
            const int64_t s = r[w] & kSlotMask;
            const float av = rf[a.Wp + w], cv = rf[2 * a.Wp + w];
            if (ok) Mc[s * a.d_v] = fmaf(av, Mc[s * a.d_v], cv * vt);
        }
        float acc = 0.f;
        for (int i = 0; i < a.R; i++) {
            const int64_t s = r[3 * a.Wp + i] & kSlotMask;
            const float qv = rf[3 * a.Wp + a.Rp + i];
            if (ok) acc = fmaf(qv, Mc[s * a.d_v], acc);
        }
        if (ok) a.y[off] = acc;
    }
}

RWArgs make_args(const Shape &s, const uint32_t *rec, const void *v, float *y, float *M)
{
    const RecLayout L(s.W, s.R);
    RWArgs a{};
    a.rec = rec;
    a.v = v;
    a.y = y;
    a.M = M;
    a.T = s.T;
    a.N = s.N();
    a.H = s.H;
    a.d_v = s.d_v;
    a.W = s.W;
    a.R = s.R;
    a.Wp = L.Wp;
    a.Rp = L.Rp;
    a.rec_dwords = L.dwords();
    return a;
}

}  // namespace

int rw_serial_depth() { return kDepth; }

namespace {

template <int LPR>
hipError_t launch_lpr(RWArgs &a, const Shape &s, bool bf16, hipStream_t st)
{
    constexpr int RPI = 64 / LPR;
    a.nslice = (s.d_v + 4 * LPR - 1) / (4 * LPR);
    a.units = (int64_t)s.B * s.H * a.nslice;
    const int64_t wgs = (a.units + 3) / 4;
    a.per_xcd = (wgs + 7) / 8;
    const dim3 grid((unsigned)(a.per_xcd * 8)), block(256);
    // references per row group; the shorter list is padded (masked references
    // cost registers only)
    const int nw = (s.W + RPI - 1) / RPI, nr = (s.R + RPI - 1) / RPI;
    const int nm = nw > nr ? nw : nr;
#define SDM_RW_CASE(NM_)                                                                        \
    if (nm <= NM_) {                                                                            \
        if (bf16)                                                                               \
            hipLaunchKernelGGL((rw_serial_kernel<LPR, NM_, NM_, kDepth, true>), grid, block, 0, \
                               st, a);                                                          \
        else                                                                                    \
            hipLaunchKernelGGL((rw_serial_kernel<LPR, NM_, NM_, kDepth, false>), grid, block,   \
                               0, st, a);                                                       \
        return hipGetLastError();                                                               \
    }
    // W, R <= 64 give nm <= LPR, so RPI * NM <= 64: every group's loads stay
    // inside the 64-entry record arrays
    SDM_RW_CASE(1)
    if constexpr (LPR >= 2) { SDM_RW_CASE(2) }
    if constexpr (LPR >= 4) { SDM_RW_CASE(4) }
    if constexpr (LPR >= 8) { SDM_RW_CASE(8) }
#undef SDM_RW_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool rw_serial_supported(const Shape &s)
{
    // the state of one chain must fit one buffer descriptor (offsets < 2^31)
    return s.d_v % 4 == 0 && (double)s.N() * s.d_v * 4.0 <= 2147483648.0;
}

hipError_t launch_rw_serial(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st)
{
    RWArgs a = make_args(s, rec, v, y, M);
    // 128-byte row slices (8 lanes x float4) give the fullest HBM bursts; with
    // fewer than 256 such units the chip is underfilled, and 32-byte slices
    // (four times the units) win.
    const int64_t units8 = (int64_t)s.B * s.H * ((s.d_v + 31) / 32);
    if (units8 >= 256) return launch_lpr<8>(a, s, bf16, st);
    return launch_lpr<2>(a, s, bf16, st);
}

hipError_t launch_rw_simple(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st)
{
    RWArgs a = make_args(s, rec, v, y, M);
    a.nslice = (s.d_v + 63) / 64;
    a.units = (int64_t)s.B * s.H * a.nslice;
    const dim3 grid((unsigned)((a.units + 3) / 4)), block(256);
    if (bf16) hipLaunchKernelGGL(rw_simple_kernel<true>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(rw_simple_kernel<false>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace sdm
