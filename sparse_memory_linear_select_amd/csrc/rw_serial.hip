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

namespace sdm {
namespace {

constexpr int kDepth = 3;  // cross-token prefetch depth of the float4 kernel

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

template <int NW, int NR, int P, bool BF16>
__global__ __launch_bounds__(256) void rw_serial_kernel(RWArgs a)
{
    __shared__ float4 ring[4][P][kMaxK][4];  // per wave: writes of the last P tokens
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    // units of one chain sit on one XCD (workgroups are dealt round-robin)
    const int64_t lwg = (int64_t)(blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
    const int64_t unit = lwg * 4 + wv;
    if (unit >= a.units) return;
    const int64_t chain = unit / a.nslice;
    const int slice = (int)(unit - chain * a.nslice);
    const int g = lane >> 2;  // row group
    const int q = lane & 3;   // float4 within the 16-column slice
    const int col = slice * 16 + q * 4;
    const bool col_ok = col < a.d_v;
    const int64_t b = chain / a.H;
    const int h = (int)(chain - b * a.H);
    const bool g_w = g * NW < a.W;  // this group has write references
    const bool g_r = g * NR < a.R;
    float *Mc = a.M + chain * a.N * a.d_v + col;
    const uint32_t *recc = a.rec + chain * a.T * a.rec_dwords;
    const int64_t T = a.T;

    uint32_t sw[2 * P][NW], sr[2 * P][NR];  // slot words, loaded 2P tokens ahead
    float4 rw[P][NW], rr[P][NR];            // gathered rows, P tokens ahead
    float ma[P][NW], mc[P][NW], mq[P][NR];  // coefficients
    float4 mv[P];                           // v_t slice

    auto load_slots = [&](int64_t t, uint32_t (&ow)[NW], uint32_t (&orr)[NR]) {
        const uint32_t *r = recc + t * a.rec_dwords;
        if (g_w) load_k<NW>(r + g * NW, ow);
        if (g_r) load_k<NR>(r + 3 * a.Wp + g * NR, orr);
    };
    auto forwarded = [](uint32_t s) {
        return (s & kFwdValid) && ((s >> kFwdDShift) & kFwdDMask) < (uint32_t)P;
    };
    auto load_rows = [&](int64_t t, const uint32_t (&iw)[NW], const uint32_t (&ir)[NR],
                         float4 (&ow)[NW], float4 (&orr)[NR], float (&oa)[NW], float (&oc)[NW],
                         float (&oq)[NR], float4 &ov) {
        const uint32_t *r = recc + t * a.rec_dwords;
        if (col_ok) {
#pragma unroll
            for (int i = 0; i < NW; i++)
                if (g * NW + i < a.W && !forwarded(iw[i]))
                    ow[i] = *reinterpret_cast<const float4 *>(Mc + (int64_t)(iw[i] & kSlotMask) * a.d_v);
#pragma unroll
            for (int i = 0; i < NR; i++)
                if (g * NR + i < a.R && !forwarded(ir[i]))
                    orr[i] = *reinterpret_cast<const float4 *>(Mc + (int64_t)(ir[i] & kSlotMask) * a.d_v);
            ov = load_v4<BF16>(a.v, (((b * T + t) * a.H) + h) * a.d_v + col);
        }
        if (g_w) {
            load_k<NW>(reinterpret_cast<const float *>(r) + a.Wp + g * NW, oa);
            load_k<NW>(reinterpret_cast<const float *>(r) + 2 * a.Wp + g * NW, oc);
        }
        if (g_r) load_k<NR>(reinterpret_cast<const float *>(r) + 3 * a.Wp + a.Rp + g * NR, oq);
    };

    // prologue
#pragma unroll
    for (int u = 0; u < 2 * P; u++)
        if (u < T) load_slots(u, sw[u], sr[u]);
#pragma unroll
    for (int u = 0; u < P; u++)
        if (u < T) load_rows(u, sw[u], sr[u], rw[u], rr[u], ma[u], mc[u], mq[u], mv[u]);

    for (int64_t t0 = 0; t0 < T; t0 += 2 * P) {
#pragma unroll
        for (int u = 0; u < 2 * P; u++) {
            const int64_t t = t0 + u;
            if (t >= T) break;
            const int pr = u % P;
            // ---- write ----
            if (col_ok) {
#pragma unroll
                for (int i = 0; i < NW; i++) {
                    const int w = g * NW + i;
                    if (w < a.W) {
                        const uint32_t s = sw[u][i];
                        float4 old = rw[pr][i];
                        if (forwarded(s)) {
                            const int d = (int)((s >> kFwdDShift) & kFwdDMask);
                            old = ring[wv][(pr - d + P) % P][(s >> kFwdWShift) & kFwdWMask][q];
                        }
                        const float av = ma[pr][i], cv = mc[pr][i];
                        float4 nv;
                        nv.x = fmaf(av, old.x, cv * mv[pr].x);
                        nv.y = fmaf(av, old.y, cv * mv[pr].y);
                        nv.z = fmaf(av, old.z, cv * mv[pr].z);
                        nv.w = fmaf(av, old.w, cv * mv[pr].w);
                        *reinterpret_cast<float4 *>(Mc + (int64_t)(s & kSlotMask) * a.d_v) = nv;
                        ring[wv][pr][w][q] = nv;
                    }
                }
            }
            wave_sync();
            // ---- read (post-write state) ----
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            if (col_ok) {
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    if (g * NR + i < a.R) {
                        const uint32_t s = sr[u][i];
                        float4 val = rr[pr][i];
                        if (forwarded(s)) {
                            const int d = (int)((s >> kFwdDShift) & kFwdDMask);
                            val = ring[wv][(pr - d + P) % P][(s >> kFwdWShift) & kFwdWMask][q];
                        }
                        const float qv = mq[pr][i];
                        acc.x = fmaf(qv, val.x, acc.x);
                        acc.y = fmaf(qv, val.y, acc.y);
                        acc.z = fmaf(qv, val.z, acc.z);
                        acc.w = fmaf(qv, val.w, acc.w);
                    }
                }
            }
#pragma unroll
            for (int m = 4; m < 64; m <<= 1) {
                acc.x += __shfl_xor(acc.x, m, 64);
                acc.y += __shfl_xor(acc.y, m, 64);
                acc.z += __shfl_xor(acc.z, m, 64);
                acc.w += __shfl_xor(acc.w, m, 64);
            }
            if (g == 0 && col_ok)
                *reinterpret_cast<float4 *>(a.y + (((b * T + t) * a.H) + h) * a.d_v + col) = acc;
            wave_sync();
            // ---- prefetch ----
            if (t + P < T)
                load_rows(t + P, sw[(u + P) % (2 * P)], sr[(u + P) % (2 * P)], rw[pr], rr[pr],
                          ma[pr], mc[pr], mq[pr], mv[pr]);
            if (t + 2 * P < T) load_slots(t + 2 * P, sw[u], sr[u]);
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

hipError_t launch_rw_serial(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st)
{
    RWArgs a = make_args(s, rec, v, y, M);
    a.nslice = (s.d_v + 15) / 16;
    a.units = (int64_t)s.B * s.H * a.nslice;
    const int64_t wgs = (a.units + 3) / 4;
    a.per_xcd = (wgs + 7) / 8;
    const dim3 grid((unsigned)(a.per_xcd * 8)), block(256);
    // W and R refs per lane group (16 groups per wave); the smaller list is
    // padded (masked references cost nothing but registers)
    const int nw = (s.W + 15) / 16, nr = (s.R + 15) / 16;
    const int nm = nw > nr ? nw : nr;
#define SDM_RW_CASE(NM_)                                                                      \
    case NM_:                                                                                 \
        if (bf16)                                                                             \
            hipLaunchKernelGGL((rw_serial_kernel<NM_, NM_, kDepth, true>), grid, block, 0, st, a); \
        else                                                                                  \
            hipLaunchKernelGGL((rw_serial_kernel<NM_, NM_, kDepth, false>), grid, block, 0, st, a); \
        break;
    switch (nm) {
        SDM_RW_CASE(1)
        SDM_RW_CASE(2)
        SDM_RW_CASE(3)
        SDM_RW_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef SDM_RW_CASE
    return hipGetLastError();
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
