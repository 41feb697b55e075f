// Backward of the SDM core on the time-parallel schedule (float32 state).
//
// Gradients of a loss L(y, M_T) with respect to k', q', v, alpha, beta and
// the initial state, with the selected slot sets held fixed (they are
// piecewise constant in k', q'; the gradient reaches k', q' through the
// softmax weights).  The forward is the one of the explainer "Sparse Delta
// Memory：通过稀疏性扩展线性 RNN 的状态容量", §3.1 steps 1-3 (the training
// discussion there asks for a memory-efficient backward and a learned
// initial state); the derivatives follow from it by the chain rule:
//   write  new = a*old + c*v, a = alpha(1 - beta k), c = beta k:
//          dold = a*g, da = <g, old>, dc = <g, v>, dv += c*g
//   read   y = sum_r q_r row_r:  g_row += q_r dy,  dq_r = <dy, row>
//   a, c -> alpha, beta, k:  dalpha = sum_w da_w (1 - beta k_w),
//          dbeta = sum_w k_w (dc_w - alpha da_w),  dk_w = beta (dc_w - alpha da_w)
//   softmax weights -> scores -> the halves of k' (q'): for slot
//          n = i*sqrtN + j, x[i] and x[sqrtN + j] receive w (dw - <w, dw>).
//
// Schedule.  A forward pass (write updates only) records, per slot written
// in an epoch, its epoch-start row at the slot's first write of the epoch
// (the tape; the rows the later writes replace are recomputed from it in the
// reverse pass with the same operations).  The tape covers one chunk of
// epochs at a time, so memory does not grow with T: a first forward pass
// keeps the state at the start of every chunk (checkpoints), then, from the
// last chunk to the first, each chunk's forward runs again from its
// checkpoint with the tape and is reversed at once.  Every chunk count gives
// the same gradients bit for bit (the recomputed forward applies the same
// operations in the same order).  The write and read events of each
// (chain, epoch) are sorted together by slot (time order within a slot,
// writes before reads at one token).  Epochs are then processed in reverse;
// per slot segment one row group walks the segment forward (rows seen by the
// reads, for dq) and backward (the adjoint g of the row, for da, dc, dv),
// then stores the slot's adjoint and its epoch-start value (state
// reconstruction without division).  Dot products are reduced over column
// slices, dv over the W writes of a token, in fixed orders: results are
// deterministic.
#include "lane_ops.h"
#include "tp_device.h"

namespace sdm {
namespace {

constexpr int kLPR = 8;  // dv reduction: 8 lanes x float4 per 128-byte column slice
constexpr int kRPI = 64 / kLPR;
constexpr int kDots = 3 * kMaxK;  // per (chain, token): da[64], dc[64], dq[64]

struct BwdArgs {
    const uint32_t *rec;     // token records
    const TPEntry *ms;       // [chain][T*(W+R)] merged sorted events, epoch regions
    float *tape;             // [chain][tapeT][W][d_v] epoch-start rows at first writes (see the segment kernel)
    int64_t tapeT, tape_t0;  // tokens per chain in the tape (one chunk), token of its first entry
    const void *v;
    const float *dy;         // [B][T][H][d_v]
    float *Mw;               // [chain][N][d_v] state: end of the current epoch -> its start
    float *G;                // [chain][N][d_v] adjoint: end of the current epoch -> its start
    float *dvbuf;            // [chain][E][W][d_v] c_k g_k of the current epoch's writes
    float *part;             // [chain][E*(W+R)][nslice][2] partial dots of the current epoch
    float *dots;             // [chain][T][kDots]
    int64_t T, N;
    int H, d_v, W, R, Wp, Rp, rec_dwords, E, nslice, sqrtN;
    int64_t chains;
};

__device__ __forceinline__ float dot4(float4 a, float4 b)
{
    return fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
}


// Segment starts of every (chain, epoch): positions p of the merged sorted
// list where the slot changes, compacted in order (a block-wide scan), and
// their number.  One 1024-thread workgroup per (chain, epoch).
__global__ __launch_bounds__(1024) void bwd_segstart_kernel(BwdArgs a, int nep, int *starts,
                                                            int *nseg)
{
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t base;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t chain = blockIdx.x / nep;
    const int ep = (int)(blockIdx.x - chain * nep);
    const int ept = a.W + a.R;
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int n = ne * ept;
    const TPEntry *se = a.ms + chain * a.T * ept + t0 * ept;
    int *st = starts + chain * a.T * ept + t0 * ept;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    if (tid == 0) base = 0;
    __syncthreads();
    for (int tb = 0; tb < n; tb += 1024) {
        const int p = tb + tid;
        const bool head = p < n && (p == 0 || se[p].slot != se[p - 1].slot);
        const uint64_t m = __ballot(head);
        if (lane == 0) wsum[wv] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t off = base;
        for (int w = 0; w < wv; w++) off += wsum[w];
        if (head) st[off + __popcll(m & below)] = p;
        __syncthreads();
        if (tid == 0) {
            uint32_t tot = 0;
            for (int w = 0; w < 16; w++) tot += wsum[w];
            base += tot;
        }
        __syncthreads();
    }
    if (tid == 0) nseg[chain * nep + ep] = (int)base;
}

// One wavefront per (chain, kSegsPerWave consecutive segments, 256-column
// group): the wave walks its segments one after the other, all 64 lanes on
// the same segment (4 columns each).  A segment's first kCache events and
// their rows -- v (write) or dy (read), and the tape row (write) -- are
// loaded in one batch; longer segments continue from memory.  Per segment:
// the epoch-start row (first write's tape entry, or the state when nothing
// writes the slot), a forward walk (the row each read sees -> dq, and the
// row each write replaces), a reverse walk (the adjoint -> da, dc, dv
// contributions), then the slot's adjoint and epoch-start state are stored.
constexpr int kCache = 4;  // events of a segment loaded in the first batch
constexpr int kSegsPerWave = 4;  // measured 4 / 8 / 16: 32.3 / 32.7 / 33.4 ms per 1.4B-style step
constexpr int kColsPerWave = 256;

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = xor_add(x, m);
    return x;
}

template <bool BF16>
__global__ __launch_bounds__(256) void bwd_segment_kernel(BwdArgs a, int ep, int nep, int nwb,
                                                          int nsg, const int *starts,
                                                          const int *nsegs)
{
    const int lane = threadIdx.x & 63;
    const uint32_t u = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sg = (int)(u % (uint32_t)nsg);
    const int wb = (int)(u / (uint32_t)nsg);
    const int64_t chain = grid_chain();
    if (chain >= a.chains || wb >= nwb) return;
    const int ept = a.W + a.R;
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int n = ne * ept;
    const int nseg = __builtin_amdgcn_readfirstlane(nsegs[chain * nep + ep]);
    const int k0 = wb * kSegsPerWave;
    if (k0 >= nseg) return;
    const int k1 = k0 + kSegsPerWave < nseg ? k0 + kSegsPerWave : nseg;
    const int col = sg * kColsPerWave + lane * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;
    const int64_t b = (uint32_t)chain / (uint32_t)a.H;  // chains < 2^32 (grid y and z)
    const int h = (int)(chain - b * a.H);
    const int64_t hd = (int64_t)a.H * a.d_v;
    const int64_t row0_off = (b * a.T * a.H + h) * a.d_v + colc;  // v, dy of token 0
    const TPEntry *se = a.ms + chain * a.T * ept + t0 * ept;
    const int *st = starts + chain * a.T * ept + t0 * ept;
    float *tape_c = a.tape + (chain * a.tapeT + (t0 - a.tape_t0)) * a.W * a.d_v + colc;
    float *part = a.part + chain * (int64_t)nsg * a.E * ept * 2 + (int64_t)sg * a.E * ept * 2;
    const rsrc_t Mr = make_rsrc(a.Mw + chain * a.N * a.d_v, (uint32_t)(a.N * a.d_v * 4));
    const rsrc_t Gr = make_rsrc(a.G + chain * a.N * a.d_v, (uint32_t)(a.N * a.d_v * 4));

    auto is_write = [](const TPEntry &x) { return (x.tw & 64u) == 0; };
    auto event_row = [&](const TPEntry &x) {  // v of a write, dy of a read
        const int64_t off = row0_off + (t0 + (x.tw >> 7)) * hd;
        float4 r;
        if ((x.tw & 64u) == 0) r = load_v<BF16>(a.v, off);
        else r = *reinterpret_cast<const float4 *>(a.dy + off);
        return r;
    };
    auto tape_row = [&](const TPEntry &x) {
        return *reinterpret_cast<const float4 *>(
            tape_c + ((int64_t)(x.tw >> 7) * a.W + (x.tw & 63u)) * a.d_v);
    };

    // the wave's segment starts (and the end of its last segment), one per
    // lane, loaded together
    const int stl = (lane <= kSegsPerWave && k0 + lane < nseg) ? st[k0 + lane] : n;
    for (int k = k0; k < k1; k++) {
        const int p0 = __builtin_amdgcn_readlane(stl, k - k0);
        const int p1 = __builtin_amdgcn_readlane(stl, k - k0 + 1);
        const int len = p1 - p0;
        const int lc = len < kCache ? len : kCache;
        const uint32_t slot = se[p0].slot;
        TPEntry e[kCache];
        float4 xv[kCache], tp[kCache];
#pragma unroll
        for (int c = 0; c < kCache; c++)
            if (c < lc) e[c] = se[p0 + c];
        // the segment's first write: its tape entry is the epoch-start row
        int firstw = -1;
#pragma unroll
        for (int c = kCache - 1; c >= 0; c--)
            if (c < lc && is_write(e[c])) firstw = c;
        float4 row0 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int c = 0; c < kCache; c++) {
            xv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < lc) xv[c] = event_row(e[c]);
            if (c == firstw) row0 = tape_row(e[c]);
        }
        const uint32_t roff = col_ok ? slot * (uint32_t)a.d_v * 4u + col * 4u : kOff;
        float4 gv = buf_load4(Gr, roff);
        bool written = firstw >= 0;
        if (firstw < 0) {
            int pw = -1;
            for (int p = p0 + lc; p < p1; p++)
                if (is_write(se[p])) {
                    pw = p;
                    break;
                }
            written = pw >= 0;
            row0 = written ? tape_row(se[pw]) : buf_load4(Mr, roff);
        }

        // forward walk: the row each read sees, and the row each write
        // replaces (recomputed with the forward's own operations, so equal
        // to it bit for bit): in registers for the cached events, in the
        // write's tape entry for the rest
        float4 cur = row0;
#pragma unroll
        for (int c = 0; c < kCache; c++) {
            tp[c] = cur;
            if (c < lc) {
                if (is_write(e[c])) {
                    cur = fma4(e[c].a, cur, e[c].c, xv[c]);
                } else {
                    const float dq = wave_sum(col_ok ? dot4(xv[c], cur) : 0.0f);
                    if (lane == 0) part[(int64_t)(p0 + c) * 2] = dq;
                }
            }
        }
        for (int p = p0 + lc; p < p1; p++) {
            const TPEntry x = se[p];
            const float4 val = event_row(x);
            if (is_write(x)) {
                if (col_ok)
                    *reinterpret_cast<float4 *>(tape_c +
                                                ((int64_t)(x.tw >> 7) * a.W + (x.tw & 63u)) *
                                                    a.d_v) = cur;
                cur = fma4(x.a, cur, x.c, val);
            } else {
                const float dq = wave_sum(col_ok ? dot4(val, cur) : 0.0f);
                if (lane == 0) part[(int64_t)p * 2] = dq;
            }
        }

        // reverse walk: the adjoint of the row
        auto rev_event = [&](const TPEntry &x, float4 val, float4 old, int p) {
            if (!is_write(x)) {  // read: g += q dy
                gv.x = fmaf(x.a, val.x, gv.x);
                gv.y = fmaf(x.a, val.y, gv.y);
                gv.z = fmaf(x.a, val.z, gv.z);
                gv.w = fmaf(x.a, val.w, gv.w);
            } else {  // write: da, dc, dv; g <- a g
                const float da = wave_sum(col_ok ? dot4(gv, old) : 0.0f);
                const float dc = wave_sum(col_ok ? dot4(gv, val) : 0.0f);
                if (lane == 0) {
                    part[(int64_t)p * 2] = da;
                    part[(int64_t)p * 2 + 1] = dc;
                }
                if (col_ok) {
                    float *dvb = a.dvbuf +
                                 ((chain * a.E + (x.tw >> 7)) * a.W + (x.tw & 63u)) * a.d_v + col;
                    *reinterpret_cast<float4 *>(dvb) =
                        make_float4(x.c * gv.x, x.c * gv.y, x.c * gv.z, x.c * gv.w);
                }
                gv = make_float4(x.a * gv.x, x.a * gv.y, x.a * gv.z, x.a * gv.w);
            }
        };
        for (int p = p1 - 1; p >= p0 + lc; p--) {  // the uncached tail, from memory
            const TPEntry x = se[p];
            const float4 val = event_row(x);
            float4 old = val;
            if (is_write(x)) old = tape_row(x);
            rev_event(x, val, old, p);
        }
#pragma unroll
        for (int c = kCache - 1; c >= 0; c--)
            if (c < lc) rev_event(e[c], xv[c], tp[c], p0 + c);
        buf_store4(gv, Gr, roff);
        if (written) buf_store4(row0, Mr, roff);  // the state at the epoch start
    }
}

// dv_t = sum over w of dvbuf[t][w] (w in order per row group, then a fixed
// butterfly across groups).  One wavefront per (chain, token, column slice).
__global__ __launch_bounds__(256) void bwd_dv_kernel(BwdArgs a, int ep, float *dv)
{
    const int lane = threadIdx.x & 63;
    const uint32_t u = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = (int)(u % (uint32_t)a.nslice);
    const int tl = (int)(u / (uint32_t)a.nslice);
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int64_t chain = grid_chain();
    if (chain >= a.chains || tl >= ne) return;
    const int g = lane / kLPR, q = lane % kLPR;
    const int col = slice * 4 * kLPR + q * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;
    const float *src = a.dvbuf + (chain * a.E + tl) * a.W * a.d_v + colc;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int w = g; w < a.W; w += kRPI) {
        const float4 x = *reinterpret_cast<const float4 *>(src + (int64_t)w * a.d_v);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
    }
#pragma unroll
    for (int m = kLPR; m < 64; m <<= 1) {
        acc.x = xor_add(acc.x, m);
        acc.y = xor_add(acc.y, m);
        acc.z = xor_add(acc.z, m);
        acc.w = xor_add(acc.w, m);
    }
    const int64_t b = (uint32_t)chain / (uint32_t)a.H;  // chains < 2^32 (grid y and z)
    const int h = (int)(chain - b * a.H);
    if (g == 0 && col_ok)
        *reinterpret_cast<float4 *>(dv + ((b * a.T + t0 + tl) * a.H + h) * a.d_v + col) = acc;
}

// Partial dots -> per (chain, token) da, dc (writes) and dq (reads): one
// thread per merged event, slices summed in order.
__global__ __launch_bounds__(256) void bwd_dots_kernel(BwdArgs a, int ep, int nsg)
{
    const int ept = a.W + a.R;
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int n = ne * ept;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.chains * n) return;
    const int64_t chain = i / n;
    const int p = (int)(i - chain * n);
    const TPEntry e = a.ms[chain * a.T * ept + t0 * ept + p];
    const float *pp = a.part + chain * (int64_t)nsg * a.E * ept * 2 + (int64_t)p * 2;
    float s0 = 0.f, s1 = 0.f;
    for (int k = 0; k < nsg; k++) {
        s0 += pp[(int64_t)k * a.E * ept * 2];
        s1 += pp[(int64_t)k * a.E * ept * 2 + 1];
    }
    float *d = a.dots + (chain * a.T + t0 + (e.tw >> 7)) * kDots;
    const int idx = (int)(e.tw & 63u);
    if (e.tw & 64u) {
        d[2 * kMaxK + idx] = s0;
    } else {
        d[idx] = s0;
        d[kMaxK + idx] = s1;
    }
}

// Per head-token and list (one wavefront each): dalpha, dbeta, the weight
// gradients, the softmax backward and the scatter onto the halves of k'
// (or q').  Every entry of the output row is a sum over the list in lane
// order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void bwd_scalar_kernel(BwdArgs a, const float *alpha,
                                                         const float *beta, float *dkp, float *dqp,
                                                         float *dalpha, float *dbeta, int64_t n_ht)
{
    // the halves' indices i, j of each selected slot (~0 past K) and its
    // score gradient, read back 4 at a time
    __shared__ __align__(16) uint32_t s1[4][kMaxK];
    __shared__ __align__(16) uint32_t s2[4][kMaxK];
    __shared__ __align__(16) float sd[4][kMaxK];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int S2 = 2 * a.sqrtN;
    for (int64_t it = (int64_t)blockIdx.x * 4 + wv; it < 2 * n_ht; it += (int64_t)gridDim.x * 4) {
        const int list = (int)(it & 1);
        const int64_t ht = it >> 1;
        const int64_t bt = ht / a.H;
        const int h = (int)(ht - bt * a.H);
        const int64_t b = bt / a.T, t = bt - b * a.T;
        const int64_t ct = (b * a.H + h) * a.T + t;
        const uint32_t *rc = a.rec + ct * a.rec_dwords;
        const float *rf = reinterpret_cast<const float *>(rc);
        const float *d = a.dots + ct * kDots;
        const int K = list ? a.R : a.W;
        const bool on = lane < K;
        float wgt = 0.f, dw = 0.f;
        uint32_t slot = 0;
        if (list == 0) {
            const float al = alpha[ht], be = beta[ht];
            float da = 0.f, dc = 0.f;
            if (on) {
                slot = rc[lane] & kSlotMask;
                wgt = rf[3 * a.Wp + 2 * a.Rp + lane];
                da = d[lane];
                dc = d[kMaxK + lane];
                dw = be * (dc - al * da);
            }
            float sa = on ? da * (1.0f - be * wgt) : 0.f;
            float sb = on ? wgt * (dc - al * da) : 0.f;
#pragma unroll
            for (int m = 32; m > 0; m >>= 1) {
                sa = xor_add(sa, m);
                sb = xor_add(sb, m);
            }
            if (lane == 0) {
                dalpha[ht] = sa;
                dbeta[ht] = sb;
            }
        } else if (on) {
            slot = rc[3 * a.Wp + lane] & kSlotMask;
            wgt = rf[3 * a.Wp + a.Rp + lane];
            dw = d[2 * kMaxK + lane];
        }
        // softmax backward: ds = w (dw - <w, dw>)
        float sw = wgt * dw;
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) sw = xor_add(sw, m);
        const float ds = on ? wgt * (dw - sw) : 0.f;
        // slot n = i*sqrtN + j: one division per selected slot, not one per
        // (slot, column) pair below
        const uint32_t si = slot / (uint32_t)a.sqrtN;
        s1[wv][lane] = on ? si : 0xFFFFFFFFu;
        s2[wv][lane] = on ? slot - si * (uint32_t)a.sqrtN : 0xFFFFFFFFu;
        sd[wv][lane] = ds;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float *out = (list ? dqp : dkp) + ht * S2;
        for (int x = lane; x < S2; x += 64) {  // x < sqrtN: first half index i; else j
            const bool first = x < a.sqrtN;
            const uint32_t want = first ? (uint32_t)x : (uint32_t)(x - a.sqrtN);
            const uint4 *part = reinterpret_cast<const uint4 *>(first ? s1[wv] : s2[wv]);
            const float4 *dsv = reinterpret_cast<const float4 *>(sd[wv]);
            float acc = 0.f;
            for (int k4 = 0; k4 < (K + 3) / 4; k4++) {  // in slot order: a deterministic sum
                const uint4 p = part[k4];
                const float4 g = dsv[k4];
                if (p.x == want) acc += g.x;
                if (p.y == want) acc += g.y;
                if (p.z == want) acc += g.z;
                if (p.w == want) acc += g.w;
            }
            out[x] = acc;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// dM0[h] = sum over b (in order) of the per-sequence initial-state gradients.
__global__ __launch_bounds__(256) void bwd_dm0_kernel(const float *G, float *dM0, int B,
                                                      int64_t per_b)
{
    // per_b = H*N*d_v is a multiple of 4 (d_v % 4 == 0): float4 accesses
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = per_b >> 2;
    const float4 *G4 = reinterpret_cast<const float4 *>(G);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int b = 0; b < B; b++) {
            const float4 g = G4[(int64_t)b * n4 + i];
            acc.x += g.x;
            acc.y += g.y;
            acc.z += g.z;
            acc.w += g.w;
        }
        reinterpret_cast<float4 *>(dM0)[i] = acc;
    }
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(float *x, int64_t n, float value)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = n >> 2;
    float4 *x4 = reinterpret_cast<float4 *>(x);
    const float4 v4 = make_float4(value, value, value, value);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        x4[i] = v4;
    for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        x[i] = value;
}

// dst <- src, n floats; float4 accesses (the callers' buffers are 16-byte
// aligned), then the tail.
__global__ __launch_bounds__(256) void bwd_copy_kernel(const float *src, float *dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = n >> 2;
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    float4 *d4 = reinterpret_cast<float4 *>(dst);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        d4[i] = s4[i];
    for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

dim3 grid_for(int64_t n, int64_t cap = 16384)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return dim3((unsigned)blocks);
}

}  // namespace

namespace {

// Layout of the backward's workspace for a given chunk count.
struct BwdLayout {
    int E, nep, chunks, per;  // epoch length, epochs, chunks, epochs per chunk
    size_t ms, mt, tape, state, dvbuf, part, dots, total;  // bytes of each region
};

BwdLayout bwd_layout(const Shape &s, int chunks)
{
    BwdLayout L{};
    const size_t chains = (size_t)s.B * s.H;
    L.E = tp_epoch_len(s);
    L.nep = (int)((s.T + L.E - 1) / L.E);
    if (chunks < 1 || chunks > L.nep) chunks = L.nep;
    L.per = (L.nep + chunks - 1) / chunks;
    L.chunks = (L.nep + L.per - 1) / L.per;
    const size_t ept = (size_t)s.W + s.R;
    const int nsg = (s.d_v + kColsPerWave - 1) / kColsPerWave;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t tape_tokens = (int64_t)L.per * L.E < s.T ? (int64_t)L.per * L.E : s.T;
    L.ms = up(chains * s.T * ept * sizeof(TPEntry));
    L.mt = up(chains * s.T * ept * 8);
    L.tape = up(chains * (size_t)tape_tokens * s.W * s.d_v * 4);
    L.state = up(chains * (size_t)s.N() * s.d_v * 4);
    L.dvbuf = up(chains * (size_t)L.E * s.W * s.d_v * 4);
    L.part = up(chains * (size_t)L.E * ept * nsg * 2 * 4);
    L.dots = up(chains * s.T * (size_t)kDots * 4);
    // merged events, 2 radix buffers, the tape, one state per chunk (the
    // first chunk's start and a checkpoint per later chunk), dv, dots
    L.total = L.ms + 2 * L.mt + L.tape + (size_t)L.chunks * L.state + L.dvbuf + L.part + L.dots;
    return L;
}

}  // namespace

int tp_backward_epochs(const Shape &s)
{
    const int E = tp_epoch_len(s);
    return (int)((s.T + E - 1) / E);
}

int tp_backward_min_chunks(const Shape &s)
{
    // fewest chunks among those that need the least memory
    const int nep = tp_backward_epochs(s);
    int best = 1;
    size_t least = bwd_layout(s, 1).total;
    for (int c = 2; c <= nep; c++) {
        const BwdLayout L = bwd_layout(s, c);
        if (L.chunks == c && L.total < least) {
            least = L.total;
            best = c;
        }
    }
    return best;
}

size_t tp_backward_workspace_bytes(const Shape &s, int chunks)
{
    return bwd_layout(s, chunks < 1 ? tp_backward_min_chunks(s) : chunks).total;
}

hipError_t launch_tp_backward(const Shape &s, int chunks, const uint32_t *rec, void *fwd_ws,
                              void *bwd_ws, const void *v, bool bf16, const float *M0,
                              const float *Minit, const float *dy, const float *dMT,
                              const float *alpha, const float *beta, float *dkp, float *dqp,
                              float *dv, float *dalpha, float *dbeta, float *dMinit, float *dM0,
                              hipStream_t st)
{
    const size_t chains = (size_t)s.B * s.H;
    const BwdLayout L = bwd_layout(s, chunks);
    const int E = L.E, nep = L.nep;
    const size_t ept = (size_t)s.W + s.R;
    const int nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    const int nsg = (s.d_v + kColsPerWave - 1) / kColsPerWave;
    char *p = static_cast<char *>(bwd_ws);
    TPEntry *ms = reinterpret_cast<TPEntry *>(p);
    p += L.ms;
    uint64_t *mtA = reinterpret_cast<uint64_t *>(p);
    p += L.mt;
    uint64_t *mtB = reinterpret_cast<uint64_t *>(p);
    p += L.mt;
    float *tape = reinterpret_cast<float *>(p);
    p += L.tape;
    float *states = reinterpret_cast<float *>(p);  // chunk c starts from states + c * nstate
    p += (size_t)L.chunks * L.state;
    float *dvbuf = reinterpret_cast<float *>(p);
    p += L.dvbuf;
    float *part = reinterpret_cast<float *>(p);
    p += L.part;
    float *dots = reinterpret_cast<float *>(p);

    const int64_t nstate = (int64_t)chains * s.N() * s.d_v;
    const size_t sstride = L.state / sizeof(float);
    auto chunk_state = [&](int c) { return states + (size_t)c * sstride; };
    hipError_t e;
    // the state the forward starts from, and the adjoint of the final state
    if (Minit) {
        hipLaunchKernelGGL(bwd_copy_kernel, grid_for(nstate), dim3(256), 0, st, Minit,
                           chunk_state(0), nstate);
        e = hipGetLastError();
    } else {
        e = launch_init(s, M0, chunk_state(0), StateFmt{}, st);
    }
    if (e != hipSuccess) return e;
    if (dMT)
        hipLaunchKernelGGL(bwd_copy_kernel, grid_for(nstate), dim3(256), 0, st, dMT, dMinit, nstate);
    else
        hipLaunchKernelGGL(bwd_fill_kernel, grid_for(nstate), dim3(256), 0, st, dMinit, nstate, 0.f);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // write events sorted per epoch, then the checkpoints: chunk c + 1 starts
    // from chunk c's start advanced over chunk c's epochs
    e = launch_tp_prepare(s, rec, fwd_ws, st, 0, -1, false);
    if (e != hipSuccess) return e;
    for (int c = 0; c + 1 < L.chunks; c++) {
        hipLaunchKernelGGL(bwd_copy_kernel, grid_for(nstate), dim3(256), 0, st, chunk_state(c),
                           chunk_state(c + 1), nstate);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = launch_tp_forward_tape(s, rec, fwd_ws, v, bf16, chunk_state(c + 1), nullptr, 0, 0,
                                   c * L.per, (c + 1) * L.per, st);
        if (e != hipSuccess) return e;
    }
    e = launch_tp_sort_merged(s, rec, fwd_ws, ms, mtA, mtB, st);
    if (e != hipSuccess) return e;

    BwdArgs a{};
    a.rec = rec;
    a.ms = ms;
    a.tape = tape;
    a.tapeT = (int64_t)L.per * E < s.T ? (int64_t)L.per * E : s.T;
    a.v = v;
    a.dy = dy;
    a.G = dMinit;
    a.dvbuf = dvbuf;
    a.part = part;
    a.dots = dots;
    a.T = s.T;
    a.N = s.N();
    a.H = s.H;
    a.d_v = s.d_v;
    a.W = s.W;
    a.R = s.R;
    const RecLayout RL(s.W, s.R);
    a.Wp = RL.Wp;
    a.Rp = RL.Rp;
    a.rec_dwords = RL.dwords();
    a.E = E;
    a.nslice = nslice;
    a.sqrtN = s.sqrtN;
    a.chains = (int64_t)chains;
    // segment starts of every (chain, epoch), into the free radix buffers
    int *starts = reinterpret_cast<int *>(mtA);
    int *nsegs = reinterpret_cast<int *>(mtB);
    hipLaunchKernelGGL(bwd_segstart_kernel, dim3((unsigned)(chains * nep)), dim3(1024), 0, st, a,
                       nep, starts, nsegs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int c = L.chunks - 1; c >= 0; c--) {
        const int ep0 = c * L.per, ep1 = (c + 1) * L.per < nep ? (c + 1) * L.per : nep;
        // the chunk's forward again, from its start, recording the tape; its
        // state buffer then holds the chunk's end state, which the reverse
        // walks back epoch by epoch
        a.Mw = chunk_state(c);
        a.tape_t0 = (int64_t)ep0 * E;
        e = launch_tp_forward_tape(s, rec, fwd_ws, v, bf16, a.Mw, tape, a.tapeT, a.tape_t0, ep0,
                                   ep1, st);
        if (e != hipSuccess) return e;
        for (int ep = ep1 - 1; ep >= ep0; ep--) {
            const int64_t t0 = (int64_t)ep * E;
            const int ne = (int)((s.T - t0) < E ? (s.T - t0) : E);
            const int nwb = (int)((ne * ept + kSegsPerWave - 1) / kSegsPerWave);  // segments <= events
            const dim3 grid = chain_grid(chains, (int64_t)nwb * nsg);
            if (bf16)
                hipLaunchKernelGGL(bwd_segment_kernel<true>, grid, dim3(256), 0, st, a, ep, nep, nwb,
                                   nsg, starts, nsegs);
            else
                hipLaunchKernelGGL(bwd_segment_kernel<false>, grid, dim3(256), 0, st, a, ep, nep, nwb,
                                   nsg, starts, nsegs);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(bwd_dv_kernel, chain_grid(chains, (int64_t)ne * nslice), dim3(256), 0,
                               st, a, ep, dv);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const int64_t nev = (int64_t)chains * ne * ept;
            hipLaunchKernelGGL(bwd_dots_kernel, dim3((unsigned)((nev + 255) / 256)), dim3(256), 0, st,
                               a, ep, nsg);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    const int64_t n_ht = s.ht();
    int64_t blocks = (2 * n_ht + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(bwd_scalar_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, alpha, beta,
                       dkp, dqp, dalpha, dbeta, n_ht);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (dM0) {
        const int64_t per_b = (int64_t)s.H * s.N() * s.d_v;
        hipLaunchKernelGGL(bwd_dm0_kernel, grid_for(per_b), dim3(256), 0, st, dMinit, dM0, s.B, per_b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sdm
