// One-token step (decode): the W writes of token t, then its R reads, which
// see those writes (the write of the explainer "Sparse Delta Memory：通过稀疏性
// 扩展线性 RNN 的状态容量", §3.1 step 2, then the read of step 3).  With one
// token there is nothing to schedule across time, so a single kernel does
// both: one wavefront per (chain, 128-byte row slice) gathers, updates and
// stores the written rows, then gathers the read rows (a read of a slot written by the same
// token finds the new row) and sums them into y.  Only the wavefront that
// wrote a row slice reads it back, so no other ordering is needed.
#include "tp_device.h"

namespace sdm {
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

// Lanes per row slice: the state's 128-byte slice, except for an E4M3 state,
// whose 128 bytes take 32 lanes; there 16 lanes (64 bytes) keep 4 row groups
// and at most 16 references per group in registers.
template <int ST>
constexpr int dec_lpr()
{
    return ST == kStateFP8 ? 16 : StateRow<ST>::kLPR;
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

}  // namespace

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
