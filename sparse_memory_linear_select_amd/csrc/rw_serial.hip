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
#include "lane_ops.h"
#include "tp_device.h"

namespace sdm {
namespace {

// Cross-token prefetch depth: the rows of token t+P are gathered while token
// t is processed (rw_serial_kernel: kDepth; rw_split_kernel, whose waves
// hold a quarter of the references each: kSplitDepth).
constexpr int kDepth = 2;
constexpr int kSplitDepth = 8;

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x of lane (lane ^ m); m is a constant once the callers' loops are unrolled
__device__ __forceinline__ float xor_get(float x, int m, int lane)
{
    if (m >= 16) {
        uint32_t lo, hi;
        pair_vals(__float_as_uint(x), m, lo, hi);
        return __uint_as_float((lane & m) ? lo : hi);
    }
    return __uint_as_float(dpp_xor(__float_as_uint(x), m));
}

struct RWArgs {
    const uint32_t *rec;
    const void *v;
    float *y, *M;
    int64_t T, N;
    int H, d_v, W, R, Wp, Rp, rec_dwords;
    int wk, rk;  // rw_split_kernel: write and read positions per wavefront
    int64_t nslice, units, per_xcd;
};

// One wavefront = one unit (chain, slice of 4*LPR columns): LPR lanes x float4
// cover one row of the slice, 64/LPR row groups take that many references at
// a time (NW write and NR read references per group per token).  The steady
// state is branch-free: masked lanes use out-of-range buffer offsets, tokens
// past the end are clamped for loads and masked for stores, so the compiler
// can keep the P-token prefetch in flight across iterations.
// WPB wavefronts per workgroup: 4 where the units give every SIMD a
// wavefront in workgroups of four, else 1.  With four, a shape with few
// units (512 at the 1.4B-style layer) filled only half of the compute
// units; single-wave workgroups spread the same waves over all of them
// (write+read 12.19 -> 11.14 ms at the 1.4B-style layer, 43.3 -> 32.8 ms
// larger state, 1681 -> 1584 ms long-context), but lose where four-wave
// workgroups already fill the chip (8B-style layer: 41.3 -> 47.8 ms).
template <int LPR, int NW, int NR, int P, bool BF16, int WPB>
__global__ __launch_bounds__(64 * WPB) void rw_serial_kernel(RWArgs a)
{
    __shared__ float4 ring[WPB][P][kMaxK][LPR];  // per wave: writes of the last P tokens
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    // the units of one chain sit on one XCD (workgroups are dealt round-robin)
    const int64_t lwg = (int64_t)(blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
    const int64_t unit = lwg * WPB + wv;
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
    const int64_t vrow0 = (b * T * a.H + h) * a.d_v + colc;  // v of token 0 of the chain
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
        ov = load_v<BF16>(a.v, vrow0 + tc * hd);
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
                acc.x = xor_add(acc.x, m);
                acc.y = xor_add(acc.y, m);
                acc.z = xor_add(acc.z, m);
                acc.w = xor_add(acc.w, m);
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

// The same token loop for shapes with few units: KS wavefronts of one
// workgroup share a unit, wave k taking write positions [k*wk, (k+1)*wk) and
// read positions [k*rk, (k+1)*rk) of every token (NW and NR per row group).
// With a single wave per unit, the 256 units of the larger-state layer or of
// the long-context sequence leave one wave per compute unit, whose token
// loop is one instruction stream; split four ways, each wave has a quarter
// of the per-token work and four waves share a compute unit.  The written
// rows go to a ring in LDS shared by the workgroup, so a forwarded row can
// come from any wave; the waves' partial sums of y meet in LDS, and wave 0
// adds them in wave order and stores y one token later.  One workgroup
// barrier per token, after its writes: the reads take same-token rows from
// the ring; a row stored before a workgroup barrier is visible to the loads
// that the other waves of the workgroup issue after it, so a prefetch may
// read a row that another wave wrote P tokens back; and the waves are never
// more than one token apart, so a ring of 2P tokens (written P or more
// tokens after its last forwarded read) and two y buffers need no other
// barrier.
template <int LPR, int NW, int NR, int P, bool BF16, int KS>
__global__ __launch_bounds__(64 * KS) void rw_split_kernel(RWArgs a)
{
    static_assert((P & (P - 1)) == 0, "ring slots are taken modulo 2P");
    __shared__ float4 ring[2 * P][kMaxK][LPR];  // writes of the last 2P tokens, all waves
    __shared__ float4 ypart[2][KS][LPR];        // partial y of each wave, by token parity
    const int lane = threadIdx.x & 63;
    const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int64_t unit = (int64_t)(blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
    if (unit >= a.units) return;  // the whole workgroup: no barrier is left waiting
    const int64_t chain = unit / a.nslice;
    const int slice = (int)(unit - chain * a.nslice);
    const int g = lane / LPR;  // row group
    const int q = lane % LPR;  // float4 within the slice
    const int col = slice * 4 * LPR + q * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;
    const int64_t b = chain / a.H;
    const int h = (int)(chain - b * a.H);
    // token numbers in 32 bits (B*T*H < 2^31); offsets from them as 32 x 32
    // -> 64-bit products
    const int T = (int)a.T;
    const uint32_t rowb = (uint32_t)a.d_v * 4u;
    const rsrc_t Mr = make_rsrc(a.M + chain * a.N * a.d_v, (uint32_t)(a.N * a.d_v * 4));
    const uint32_t *recc = a.rec + chain * a.T * a.rec_dwords;
    const uint32_t recd = (uint32_t)a.rec_dwords;
    const uint32_t hd = (uint32_t)a.H * (uint32_t)a.d_v;  // stride of one token in v and y
    const int64_t vrow0 = (b * a.T * a.H + h) * a.d_v + colc;
    float *ybase = a.y + (b * a.T * a.H + h) * a.d_v;
    // positions of this lane's references; groups past the wave's share load
    // the share's last group (record reads stay inside the 64-entry arrays)
    const bool gw = g * NW < a.wk, gr = g * NR < a.rk;
    const int lw = k * a.wk + (gw ? g : a.wk / NW - 1) * NW;
    const int lr = k * a.rk + (gr ? g : a.rk / NR - 1) * NR;
    bool pw[NW], okw[NW], okr[NR];
#pragma unroll
    for (int i = 0; i < NW; i++) {
        pw[i] = gw & (lw + i < a.W);  // a position of this wave's share
        okw[i] = col_ok & pw[i];
    }
#pragma unroll
    for (int i = 0; i < NR; i++) okr[i] = col_ok & gr & (lr + i < a.R);

    uint32_t sw[2 * P][NW], sr[2 * P][NR];
    float4 rw[P][NW], rr[P][NR];
    // coefficients and v of the next kQ tokens: their loads need less lead
    // than the row gathers (and each token's are issued before its rows,
    // so waiting for them never waits for rows issued later)
    constexpr int kQ = 2;
    static_assert((2 * P) % kQ == 0, "coefficient slots are taken modulo kQ");
    float ma[kQ][NW], mc[kQ][NW], mq[kQ][NR];
    float4 mv[kQ];

    auto clampt = [&](int t) { return (uint32_t)(t < 0 ? 0 : (t < T ? t : T - 1)); };
    auto fwd = [](uint32_t s) {
        return ((s & kFwdValid) != 0) & (((s >> kFwdDShift) & kFwdDMask) < (uint32_t)P);
    };
    auto load_slots = [&](int t, uint32_t (&ow)[NW], uint32_t (&orr)[NR]) {
        const uint32_t *r = recc + (uint64_t)clampt(t) * recd;
        load_k<NW>(r + lw, ow);
        load_k<NR>(r + 3 * a.Wp + lr, orr);
    };
    auto load_rows = [&](const uint32_t (&iw)[NW], const uint32_t (&ir)[NR], float4 (&ow)[NW],
                         float4 (&orr)[NR]) {
#pragma unroll
        for (int i = 0; i < NW; i++)
            ow[i] = buf_load4(Mr, (okw[i] & !fwd(iw[i])) ? (iw[i] & kSlotMask) * rowb + col * 4u : kOff);
#pragma unroll
        for (int i = 0; i < NR; i++)
            orr[i] = buf_load4(Mr, (okr[i] & !fwd(ir[i])) ? (ir[i] & kSlotMask) * rowb + col * 4u : kOff);
    };
    auto load_coef = [&](int t, float (&oa)[NW], float (&oc)[NW], float (&oq)[NR], float4 &ov) {
        const uint32_t tc = clampt(t);
        ov = load_v<BF16>(a.v, vrow0 + (int64_t)((uint64_t)tc * hd));
        const float *r = reinterpret_cast<const float *>(recc + (uint64_t)tc * recd);
        load_k<NW>(r + a.Wp + lw, oa);
        load_k<NW>(r + 2 * a.Wp + lw, oc);
        load_k<NR>(r + 3 * a.Wp + a.Rp + lr, oq);
    };

#pragma unroll
    for (int u = 0; u < 2 * P; u++) {
#pragma unroll
        for (int i = 0; i < NW; i++) sw[u][i] = 0;
#pragma unroll
        for (int i = 0; i < NR; i++) sr[u][i] = 0;
    }
#pragma unroll
    for (int u = 0; u < P; u++) {
#pragma unroll
        for (int i = 0; i < NW; i++) rw[u][i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < NR; i++) rr[u][i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kQ; u++) {
        mv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < NW; i++) {
            ma[u][i] = 0.f;
            mc[u][i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < NR; i++) mq[u][i] = 0.f;
    }

    // wave 0 stores y of the previous token (sum of the waves' partials, in
    // wave order)
    auto store_y = [&](const rsrc_t &Yr, int slot, uint32_t off, bool live) {
        if (k == 0 && g == 0) {
            float4 ys = ypart[slot][0][q];
#pragma unroll
            for (int j = 1; j < KS; j++) {
                const float4 p = ypart[slot][j][q];
                ys.x += p.x;
                ys.y += p.y;
                ys.z += p.z;
                ys.w += p.w;
            }
            buf_store4(ys, Yr, (col_ok & live) ? off : kOff);
        }
    };

    int t0 = -2 * P;
    for (; t0 < T; t0 += 2 * P) {
        // y of tokens t0-1 .. t0+2P-2 through a descriptor based at token
        // t0-1 (only offsets of tokens in [0, T) are ever used)
        const rsrc_t Yr = make_rsrc(ybase + (int64_t)(t0 - 1) * hd, 2 * P * hd * 4);
#pragma unroll
        for (int u = 0; u < 2 * P; u++) {
            const int pr = u % P, cq = u % kQ;
            const bool live = (t0 + u >= 0) & (t0 + u < T);
            // ---- this wave's writes ----
#pragma unroll
            for (int i = 0; i < NW; i++) {
                const uint32_t s = sw[u][i];
                const bool f = fwd(s);
                const int d = f ? (int)((s >> kFwdDShift) & kFwdDMask) : 0;
                const int wp = f ? (int)((s >> kFwdWShift) & kFwdWMask) : 0;
                const float4 fv = ring[(u - d) & (2 * P - 1)][wp][q];
                const float4 old = f ? fv : rw[pr][i];
                const float4 nv = fma4(ma[cq][i], old, mc[cq][i], mv[cq]);
                buf_store4(nv, Mr, (okw[i] & live) ? (s & kSlotMask) * rowb + col * 4u : kOff);
                if (pw[i]) ring[u][lw + i][q] = nv;
            }
            __syncthreads();
            store_y(Yr, (u + 1) & 1, ((uint32_t)u * hd + (uint32_t)col) * 4u,
                    (t0 + u - 1 >= 0) & (t0 + u - 1 < T));
            // ---- this wave's reads of the post-write state ----
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < NR; i++) {
                // a masked reference holds a copy of a live one's slot word:
                // never forwarded, its (not loaded) row reads as zero
                const uint32_t s = sr[u][i];
                const bool f = fwd(s) & okr[i];
                const int d = f ? (int)((s >> kFwdDShift) & kFwdDMask) : 0;
                const int wp = f ? (int)((s >> kFwdWShift) & kFwdWMask) : 0;
                const float4 fv = ring[(u - d) & (2 * P - 1)][wp][q];
                const float4 val = f ? fv : rr[pr][i];
                const float qv = mq[cq][i];
                acc.x = fmaf(qv, val.x, acc.x);
                acc.y = fmaf(qv, val.y, acc.y);
                acc.z = fmaf(qv, val.z, acc.z);
                acc.w = fmaf(qv, val.w, acc.w);
            }
            // sum over the row groups, transposed: each step hands the
            // partner the components it does not keep, so that afterwards
            // lane (g, q) holds component 2 (g & 1) + ((g >> 1) & 1) of the
            // wave's sum for float4 q (6 lane moves instead of 4 per step)
            const bool b0 = (g & 1) != 0, b1 = (g & 2) != 0;
            float k0 = b0 ? acc.z : acc.x, k1 = b0 ? acc.w : acc.y;
            k0 += xor_get(b0 ? acc.x : acc.z, LPR, lane);
            k1 += xor_get(b0 ? acc.y : acc.w, LPR, lane);
            float kc = b1 ? k1 : k0;
            kc += xor_get(b1 ? k0 : k1, 2 * LPR, lane);
#pragma unroll
            for (int m = 4 * LPR; m < 64; m <<= 1) kc = xor_add(kc, m);
            if (g < 4) reinterpret_cast<float *>(&ypart[u & 1][k][q])[2 * (g & 1) + (g >> 1)] = kc;
            // ---- prefetch: coefficients and v of token t+kQ, rows of token
            // t+P, slot words of token t+2P ----
            load_coef(t0 + u + kQ, ma[cq], mc[cq], mq[cq], mv[cq]);
            load_rows(sw[(u + P) % (2 * P)], sr[(u + P) % (2 * P)], rw[pr], rr[pr]);
            load_slots(t0 + u + 2 * P, sw[u], sr[u]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the last trip's last token (t0 - 1 now) has no next token to store its y
    __syncthreads();
    const rsrc_t Yr = make_rsrc(ybase + (int64_t)(t0 - 1) * hd, hd * 4);
    store_y(Yr, 1, (uint32_t)col * 4u, t0 - 1 < T);
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

namespace {

template <int LPR, int WPB>
hipError_t launch_lpr(RWArgs &a, const Shape &s, bool bf16, hipStream_t st)
{
    constexpr int RPI = 64 / LPR;
    const int64_t wgs = (a.units + WPB - 1) / WPB;
    a.per_xcd = (wgs + 7) / 8;
    const dim3 grid((unsigned)(a.per_xcd * 8)), block(64 * WPB);
    // references per row group; the shorter list is padded (masked references
    // cost registers only)
    const int nw = (s.W + RPI - 1) / RPI, nr = (s.R + RPI - 1) / RPI;
    const int nm = nw > nr ? nw : nr;
#define SDM_RW_CASE(NM_)                                                                        \
    if (nm <= NM_) {                                                                            \
        if (bf16)                                                                               \
            hipLaunchKernelGGL((rw_serial_kernel<LPR, NM_, NM_, kDepth, true, WPB>), grid,     \
                               block, 0, st, a);                                                \
        else                                                                                    \
            hipLaunchKernelGGL((rw_serial_kernel<LPR, NM_, NM_, kDepth, false, WPB>), grid,    \
                               block, 0, st, a);                                                \
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

// rw_split_kernel with KS waves per unit: each wave takes ceil(W / KS)
// write and ceil(R / KS) read positions (rounded up to whole row-group
// loads), NM per row group
template <int LPR, int KS>
hipError_t launch_split(RWArgs &a, const Shape &s, bool bf16, hipStream_t st)
{
    constexpr int G = 64 / LPR;
    const int pw = (s.W + KS - 1) / KS, pr = (s.R + KS - 1) / KS;
    const int nm = ((pw > pr ? pw : pr) + G - 1) / G;
    a.per_xcd = (a.units + 7) / 8;
    const dim3 grid((unsigned)(a.per_xcd * 8)), block(64 * KS);
#define SDM_SPLIT_CASE(NM_)                                                                     \
    if (nm <= NM_) {                                                                            \
        a.wk = (pw + NM_ - 1) / NM_ * NM_;                                                      \
        a.rk = (pr + NM_ - 1) / NM_ * NM_;                                                      \
        if (KS * a.wk > kMaxK || KS * a.rk > kMaxK) return hipErrorInvalidValue;               \
        if (bf16)                                                                               \
            hipLaunchKernelGGL((rw_split_kernel<LPR, NM_, NM_, kSplitDepth, true, KS>), grid,  \
                               block, 0, st, a);                                                \
        else                                                                                    \
            hipLaunchKernelGGL((rw_split_kernel<LPR, NM_, NM_, kSplitDepth, false, KS>), grid, \
                               block, 0, st, a);                                                \
        return hipGetLastError();                                                               \
    }
    SDM_SPLIT_CASE(1)
    SDM_SPLIT_CASE(2)
#undef SDM_SPLIT_CASE
    return hipErrorInvalidValue;
}

// Which kernel runs a shape: 128-byte row slices (8 lanes x float4) give the
// fullest HBM bursts; where those units give every SIMD a wave in
// workgroups of four, one wave per unit (rw_serial_kernel); else the split
// kernel with ks waves per unit, and 32-byte slices (four times the units)
// where 128-byte ones leave compute units without a unit.
struct SerialPlan {
    int lpr, ks;  // lanes per row slice; waves per unit (1: rw_serial_kernel)
};

SerialPlan serial_plan(const Shape &s)
{
    const int64_t units8 = (int64_t)s.B * s.H * ((s.d_v + 31) / 32);
    const int64_t cus = compute_units();
    if (units8 >= 4 * cus) return {8, 1};
    return {units8 >= cus ? 8 : 2, 4};
}

}  // namespace

int rw_serial_depth(const Shape &s) { return serial_plan(s).ks > 1 ? kSplitDepth : kDepth; }

bool rw_serial_supported(const Shape &s)
{
    // the state of one chain must fit one buffer descriptor (offsets < 2^31)
    return s.d_v % 4 == 0 && (double)s.N() * s.d_v * 4.0 <= 2147483648.0;
}

hipError_t launch_rw_serial(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st)
{
    RWArgs a = make_args(s, rec, v, y, M);
    const SerialPlan p = serial_plan(s);
    a.nslice = (s.d_v + 4 * p.lpr - 1) / (4 * p.lpr);
    a.units = (int64_t)s.B * s.H * a.nslice;
#define SDM_PLAN_CASE(LPR_, KS_) \
    if (p.lpr == LPR_ && p.ks == KS_) return launch_split<LPR_, KS_>(a, s, bf16, st);
    if (p.ks == 1) return launch_lpr<8, 4>(a, s, bf16, st);
    SDM_PLAN_CASE(8, 4)
    SDM_PLAN_CASE(2, 4)
#undef SDM_PLAN_CASE
    return hipErrorInvalidValue;
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
