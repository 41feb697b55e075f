// Time-parallel write/read schedule of the SDM core.
//
// The recurrence of one chain (sequence b, head h) is, per slot, a sequence of
// affine maps row <- a*row + c*v_t (a = alpha_t(1 - beta_t k), c = beta_t k:
// the forget gate and delta write of the explainer "Sparse Delta Memory：通过
// 稀疏性扩展线性 RNN 的状态容量", §3.1 step 2), and a read at token t sees the
// row after every write at a token <= t (§3.1 step 3).  Slots never interact,
// so the tokens are cut into epochs of E tokens and, per epoch:
//
//   sort     (before the recurrence) the E*W write events of the epoch are
//            sorted by slot with a stable LSD radix sort, so each slot's
//            writes form one segment in time order;
//   plan     every read gets the weight of its slot's epoch-start row and
//            the (token, weight) pairs of the v rows its in-epoch writes
//            added (the composed affine map, scaled by the read weight q);
//   read     y_t = weighted sum of epoch-start rows and v rows, all gathers
//            independent of each other;
//   update   the first event of each slot's segment loads the row once,
//            applies all of the segment's writes in time order and stores it
//            once.
//
// Within an epoch everything is parallel; epochs follow each other in stream
// order (read of epoch e, update of e, read of e+1, ...).  Each row value is
// produced by the same float32 operations, in the same order, as in the
// token-serial schedule, so both schedules give identical M; y agrees to
// float32 rounding (its terms are grouped differently).
#include "tp_device.h"

namespace sdm {
namespace {

constexpr int kSortThreads = 1024;
constexpr int kMaxEpoch = 4096;            // tokens per epoch
constexpr int kMaxEpochEvents = 1 << 18;   // write events per (chain, epoch)
constexpr int kCntBits = 13;               // replay link: count < 2^13, position < 2^19
constexpr uint32_t kReplayFlag = 1u << 31;  // in npair: the token has replay links
static_assert(kMaxEpoch < (1 << kCntBits), "a slot is written at most once per token");

struct TPArgs {
    const uint32_t *rec;  // token records (slots, coefficients)
    TPEntry *sorted;      // [chain][T*W] sorted write events, epoch regions
    uint64_t *tmpA, *tmpB;  // [chain][T*W] radix ping-pong (key << 32 | event)
    uint16_t *ckey;       // [chain][T*W] coarse keys of the sorted events (slot >> kshift)
    uint32_t *rlink;      // [chain][T][kMaxK] replay links: (first << kCntBits) | count
    float *rwt;           // [chain][T][kMaxK] weight of each read's epoch-start row
    uint32_t *npair;      // [chain][T] pairs in use (| kReplayFlag: some read replays)
    uint2 *pairs;         // [chain][T][P] (token in epoch, weight) of v rows to add
    int P;                // pair capacity per token
    const void *v;
    float *y;
    void *M;  // float32 or bfloat16 state
    int64_t T, N;
    int H, d_v, W, R, Wp, Rp, rec_dwords;
    int E, nepoch, passes, kshift;
    int ep0, nrun;  // sort/link launches: epochs [ep0, ep0 + nrun)
    int64_t chains;
    float *tape;    // backward's forward pass: [chain][T][W][d_v] row each write replaced
};

// Where a sort writes: the forward sorts the W write events of each token;
// the backward sorts them together with the R read events (W + R per token).
struct SortIO {
    TPEntry *out;           // [chain][T * per_token] sorted entries, epoch regions
    uint64_t *tmpA, *tmpB;  // radix ping-pong, same layout
    uint16_t *ckey;         // coarse keys (forward only)
};

// ------------------------------------------------------------------ sort

constexpr int kDigitBits = 9;                  // radix digit: 512 buckets
constexpr int kBuckets = 1 << kDigitBits;
constexpr int kWaves = kSortThreads / 64;

// Stable LSD radix sort of one epoch's write events by slot (one workgroup per
// (chain, epoch)).  Events are numbered j = token_in_epoch * W + w, so the
// input order is time order and stability keeps each slot's writes in time
// order.  The last pass writes the 16-byte entries and a 16-bit coarse key
// (slot >> kshift) per entry for the link search.
template <bool MERGED>
__global__ __launch_bounds__(kSortThreads) void tp_sort_kernel(TPArgs a, SortIO io)
{
    const int ept = MERGED ? a.W + a.R : a.W;  // events per token
    __shared__ uint32_t bins[kBuckets];
    __shared__ uint32_t wcnt[kWaves][kBuckets];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int64_t chain = blockIdx.x / a.nrun;
    const int ep = a.ep0 + (int)(blockIdx.x - chain * a.nrun);
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);  // tokens in this epoch
    const int n = ne * ept;                                      // events
    const int64_t base = chain * a.T * ept + t0 * ept;          // epoch region
    const uint32_t *recc = a.rec + (chain * a.T + t0) * a.rec_dwords;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int p = 0; p < a.passes; p++) {
        const int shift = kDigitBits * p;
        const uint64_t *src = (p & 1) ? io.tmpA + base : io.tmpB + base;  // unused when p == 0
        uint64_t *dst = (p & 1) ? io.tmpB + base : io.tmpA + base;
        const bool last = p == a.passes - 1;
        auto item = [&](int j) -> uint64_t {  // (slot << 32) | event j
            if (p == 0) {
                const int tl = j / ept, k = j - tl * ept;  // k >= W: read k - W
                const int col = (MERGED && k >= a.W) ? 3 * a.Wp + (k - a.W) : k;
                return ((uint64_t)(recc[(int64_t)tl * a.rec_dwords + col] & kSlotMask) << 32) |
                       (uint32_t)j;
            }
            return src[j];
        };
        // histogram of this digit
        for (int k = tid; k < kBuckets; k += kSortThreads) bins[k] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kSortThreads)
            atomicAdd(&bins[(uint32_t)(item(j) >> (32 + shift)) & (kBuckets - 1)], 1u);
        __syncthreads();
        if (wv == 0) {  // exclusive scan of the buckets, kBuckets/64 per lane
            constexpr int PER = kBuckets / 64;
            uint32_t c[PER], sum = 0;
            for (int k = 0; k < PER; k++) {
                c[k] = bins[lane * PER + k];
                sum += c[k];
            }
            uint32_t incl = sum;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = (uint32_t)__shfl_up((int)incl, o, 64);
                if (lane >= o) incl += t;
            }
            uint32_t run = incl - sum;
            for (int k = 0; k < PER; k++) {
                bins[lane * PER + k] = run;
                run += c[k];
            }
        }
        __syncthreads();
        // stable scatter, one tile of kSortThreads events at a time
        for (int tb = 0; tb < n; tb += kSortThreads) {
            const int j = tb + tid;
            const bool valid = j < n;
            const uint64_t it = valid ? item(j) : 0;
            const uint32_t dg = (uint32_t)(it >> (32 + shift)) & (kBuckets - 1);
            for (int k = tid; k < kWaves * kBuckets; k += kSortThreads) (&wcnt[0][0])[k] = 0;
            uint64_t peers = __ballot(valid);  // lanes of this wave with the same digit
            for (int bit = 0; bit < kDigitBits; bit++) {
                const uint64_t m = __ballot((dg >> bit) & 1u);
                peers &= ((dg >> bit) & 1u) ? m : ~m;
            }
            const uint32_t rank = (uint32_t)__popcll(peers & lanes_below);
            __syncthreads();
            if (valid && rank == 0) wcnt[wv][dg] = (uint32_t)__popcll(peers);
            __syncthreads();
            for (int d = tid; d < kBuckets; d += kSortThreads) {  // per digit, in wave order
                uint32_t run = bins[d];
                for (int w = 0; w < kWaves; w++) {
                    const uint32_t c = wcnt[w][d];
                    wcnt[w][d] = run;
                    run += c;
                }
                bins[d] = run;
            }
            __syncthreads();
            if (valid) {
                const uint32_t pos = wcnt[wv][dg] + rank;
                if (!last) {
                    dst[pos] = it;
                } else {  // final order: the 16-byte entries and the coarse keys
                    const uint32_t ev = (uint32_t)it;
                    const int tl = (int)(ev / (uint32_t)ept), k = (int)(ev - tl * ept);
                    const float *rf = reinterpret_cast<const float *>(recc + (int64_t)tl * a.rec_dwords);
                    TPEntry e;
                    e.slot = (uint32_t)(it >> 32);
                    if (!MERGED) {  // write w = k: (token << 6) | w, a, c
                        e.tw = ((uint32_t)tl << 6) | (uint32_t)k;
                        e.a = rf[a.Wp + k];
                        e.c = rf[2 * a.Wp + k];
                    } else if (k < a.W) {  // write: (token << 7) | w, a, c
                        e.tw = ((uint32_t)tl << 7) | (uint32_t)k;
                        e.a = rf[a.Wp + k];
                        e.c = rf[2 * a.Wp + k];
                    } else {  // read r: (token << 7) | 64 | r, q, 0
                        e.tw = ((uint32_t)tl << 7) | 64u | (uint32_t)(k - a.W);
                        e.a = rf[3 * a.Wp + a.Rp + (k - a.W)];
                        e.c = 0.0f;
                    }
                    io.out[base + pos] = e;
                    if (!MERGED) io.ckey[base + pos] = (uint16_t)(e.slot >> a.kshift);
                }
            }
            __syncthreads();
        }
    }
}

// Read plan of one (chain, epoch).  A read of slot s at token t sees the
// epoch-start row of s after the epoch's writes to s at tokens <= t, i.e.
// (in time order k = 1..m, row <- a_k row + c_k v_k)
//     row_t = A row_0 + sum_k C_k v_k,   A = prod_k a_k,  C_k = c_k prod_{l>k} a_l,
// so q * row_t is a weighted sum of one epoch-start row and m rows of v.  Per
// token, the read kernel gets the row weights q*A and a list of
// (token, q*C_k) pairs; reads whose pairs do not fit the token's capacity P
// keep weight q and a link (first write, count) that the read kernel replays.
// The sorted writes of s form one segment (time order); the coarse keys
// (slot >> kshift) of every stride-th sorted write sit in LDS (at most
// 64 KiB): a binary search there brackets the slot, a short forward scan of
// the entries finds the exact range.  One wavefront per token: lane r takes
// read r, a prefix sum over the lanes places the pairs.
__global__ __launch_bounds__(kSortThreads) void tp_link_kernel(TPArgs a, int stride, int exact)
{
    extern __shared__ uint16_t ck[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t chain = blockIdx.x / a.nrun;
    const int ep = a.ep0 + (int)(blockIdx.x - chain * a.nrun);
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int n = ne * a.W;
    const int ns = (n + stride - 1) / stride;
    const int64_t base = chain * a.T * a.W + t0 * a.W;
    const uint32_t *recc = a.rec + (chain * a.T + t0) * a.rec_dwords;
    const TPEntry *se = a.sorted + base;
    // exact (every write sampled, keys = slots): the token of every sorted
    // write sits in LDS as well, and the searches never touch memory
    uint16_t *tk = ck + ns;
    for (int k = tid; k < ns; k += kSortThreads) {
        ck[k] = a.ckey[base + (int64_t)k * stride];
        if (exact) tk[k] = (uint16_t)(se[k].tw >> 6);
    }
    __syncthreads();
    for (int tl = tid >> 6; tl < ne; tl += kSortThreads / 64) {  // wave-uniform token
        const uint32_t *rc = recc + (int64_t)tl * a.rec_dwords;
        const bool real = lane < a.R;
        int j = 0, cnt = 0;
        float q = 0.0f;
        if (real) {
            const uint32_t s = rc[3 * a.Wp + lane] & kSlotMask;
            q = __uint_as_float(rc[3 * a.Wp + a.Rp + lane]);
            const uint32_t c = s >> a.kshift;
            int lo = 0, hi = ns;  // first sample with coarse key >= c
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (ck[mid] < c) lo = mid + 1;
                else hi = mid;
            }
            int l2;  // past the writes of s at tokens <= tl
            if (exact) {
                j = lo;
                l2 = j;
                while (l2 < n && ck[l2] == s && (int)tk[l2] <= tl) l2++;
            } else {
                // the sample before it has a smaller slot, so the slot's first
                // entry follows it; both scans look at two entries per round trip
                j = lo > 0 ? (lo - 1) * stride + 1 : 0;
                while (j < n) {
                    const uint32_t s0 = se[j].slot, s1 = se[j + 1 < n ? j + 1 : j].slot;
                    if (s0 >= s) break;
                    if (++j >= n || s1 >= s) break;
                    j++;
                }
                l2 = j;
                while (l2 < n) {
                    const TPEntry e0 = se[l2], e1 = se[l2 + 1 < n ? l2 + 1 : l2];
                    if (e0.slot != s || (int)(e0.tw >> 6) > tl) break;
                    if (++l2 >= n || e1.slot != s || (int)(e1.tw >> 6) > tl) break;
                    l2++;
                }
            }
            cnt = l2 - j;
        }
        // exclusive prefix sum of cnt over the lanes: this read's first pair
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, 64);
            if (lane >= o) incl += u;
        }
        const int off = incl - cnt;
        const bool fits = off + cnt <= a.P;
        const int64_t ct = chain * a.T + t0 + tl;
        uint2 *pp = a.pairs + ct * a.P;
        float w = q;
        if (cnt > 0 && fits) {
            float A = 1.0f;  // product of the a's after the current write
            for (int k = cnt - 1; k >= 0; k--) {
                const TPEntry e = se[j + k];
                pp[off + k] = make_uint2(e.tw >> 6, __float_as_uint(q * (e.c * A)));
                A *= e.a;
            }
            w = q * A;
        }
        a.rwt[ct * kMaxK + lane] = w;
        // j < n <= kMaxEpochEvents when cnt > 0
        a.rlink[ct * kMaxK + lane] = (cnt > 0 && !fits) ? (((uint32_t)j << kCntBits) | cnt) : 0u;
        // the reads that fit are a prefix of the lanes: their pairs are [0, npair)
        const unsigned long long over = __ballot(cnt > 0 && !fits);
        const int first_over = over ? __builtin_ctzll(over) : 63;
        const int off_over = __shfl(off, first_over, 64);
        const int total = __shfl(incl, 63, 64);
        // bit 31: some read of this token replays its writes
        if (lane == 0) a.npair[ct] = over ? ((uint32_t)off_over | kReplayFlag) : (uint32_t)total;
    }
}

// ------------------------------------------------------------------ read

// One wavefront per (chain, token of the epoch, 32-column slice).  With the
// read plan, y_t = sum_r w_r row_r + sum_j u_j v_(t_j): the 8 row groups take
// 8 reads at a time (epoch-start rows, as in the serial kernel), then the
// token's v pairs 8 at a time.  Every load depends only on the plan, so all
// of them can be in flight together; reads that overflowed the plan replay
// their writes from the sorted events.
#ifndef SDM_TP_PAIR_BATCH
#define SDM_TP_PAIR_BATCH 4
#endif
constexpr int kPairBatch = SDM_TP_PAIR_BATCH;  // v pairs per row group in flight

template <int NR, bool BF16, bool SB>
__global__ __launch_bounds__(256) void tp_read_kernel(TPArgs a, int ep, int nslice)
{
    using S = StateRow<SB>;
    constexpr int kLPR = S::kLPR, kRPI = 64 / kLPR;
    const int lane = threadIdx.x & 63;
    const int64_t chain = grid_chain();
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const uint32_t u = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (chain >= a.chains || u >= (uint32_t)(ne * nslice)) return;
    const int slice = (int)(u % (uint32_t)nslice);
    const int tl = (int)(u / (uint32_t)nslice);
    const int64_t t = t0 + tl;
    const int64_t ct = chain * a.T + t;
    const int g = lane / kLPR, q = lane % kLPR;
    const int col = slice * 4 * kLPR + q * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;
    // chains < 2^32 (the grid's y and z), so 32-bit division
    const int64_t b = (uint32_t)chain / (uint32_t)a.H;
    const int h = (int)(chain - b * a.H);
    const int64_t hd = (int64_t)a.H * a.d_v;
    const int64_t vrow0 = (b * a.T * a.H + h) * a.d_v + colc;  // v of token 0 of the chain
    const rsrc_t Mr = make_rsrc(static_cast<char *>(a.M) + chain * a.N * a.d_v * S::kElem,
                                (uint32_t)(a.N * a.d_v * S::kElem));
    const uint32_t rowb = (uint32_t)a.d_v * S::kElem;
    const uint32_t *rc = a.rec + ct * a.rec_dwords;
    const TPEntry *se = a.sorted + chain * a.T * a.W + t0 * a.W;
    const uint2 *pp = a.pairs + ct * a.P;
    const uint32_t npw = __builtin_amdgcn_readfirstlane(a.npair[ct]);
    const int np = (int)(npw & ~kReplayFlag);

    // lane q of row group g holds the slot word and weight of reference
    // g*NR + q (q < NR); the group reads them back with in-group broadcasts
    const bool mine = (q < NR) & (g * NR + q < a.R);
    const uint32_t sl_mine = mine ? rc[3 * a.Wp + g * NR + q] : 0u;
    const float wr_mine = mine ? a.rwt[ct * kMaxK + g * NR + q] : 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!(npw & kReplayFlag)) {
        // every row gather at once, then the weighted sum
        typename S::Raw row[NR];
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const uint32_t sl = group_bcast<kLPR>(sl_mine, i);
            const bool ok = col_ok & (g * NR + i < a.R);
            row[i] = S::load_raw(Mr, ok ? (sl & kSlotMask) * rowb + col * S::kElem : kOff);
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            // masked references have weight 0 and a zero row
            const float4 rv = S::widen(row[i]);
            const float wr = __uint_as_float(group_bcast<kLPR>(__float_as_uint(wr_mine), i));
            acc.x = fmaf(wr, rv.x, acc.x);
            acc.y = fmaf(wr, rv.y, acc.y);
            acc.z = fmaf(wr, rv.z, acc.z);
            acc.w = fmaf(wr, rv.w, acc.w);
        }
    } else {
        // rare: some reads of this token replay the writes their pairs could
        // not hold; one reference at a time
        const uint32_t *lkp = a.rlink + ct * kMaxK + g * NR;
#pragma unroll 1
        for (int i = 0; i < NR; i++) {
            const uint32_t sl = group_bcast<kLPR>(sl_mine, i);
            const bool ok = col_ok & (g * NR + i < a.R);
            float4 rv = S::load(Mr, ok ? (sl & kSlotMask) * rowb + col * S::kElem : kOff);
            // links exist only for the R real references; zero unless the plan overflowed
            const uint32_t l = (g * NR + i < a.R) ? lkp[i] : 0u;
            const int first = (int)(l >> kCntBits), cnt = (int)(l & ((1u << kCntBits) - 1u));
            for (int k = 0; k < cnt; k++) {  // writes of this slot earlier in the epoch
                const TPEntry e = se[first + k];
                const float4 vv = load_v<BF16>(a.v, vrow0 + (t0 + (e.tw >> 6)) * hd);
                rv = S::round(fma4(e.a, rv, e.c, vv));
            }
            const float wr = __uint_as_float(group_bcast<kLPR>(__float_as_uint(wr_mine), i));
            acc.x = fmaf(wr, rv.x, acc.x);
            acc.y = fmaf(wr, rv.y, acc.y);
            acc.z = fmaf(wr, rv.z, acc.z);
            acc.w = fmaf(wr, rv.w, acc.w);
        }
    }
    for (int j0 = 0; j0 < np; j0 += kRPI * kPairBatch) {
        uint2 pr[kPairBatch];
        float4 vv[kPairBatch];
#pragma unroll
        for (int u = 0; u < kPairBatch; u++) {
            const int j = j0 + u * kRPI + g;
            pr[u] = j < np ? pp[j] : make_uint2(0u, 0u);  // weight 0 past the end
        }
#pragma unroll
        for (int u = 0; u < kPairBatch; u++) vv[u] = load_v<BF16>(a.v, vrow0 + (t0 + pr[u].x) * hd);
#pragma unroll
        for (int u = 0; u < kPairBatch; u++) {
            const float wgt = __uint_as_float(pr[u].y);
            acc.x = fmaf(wgt, vv[u].x, acc.x);
            acc.y = fmaf(wgt, vv[u].y, acc.y);
            acc.z = fmaf(wgt, vv[u].z, acc.z);
            acc.w = fmaf(wgt, vv[u].w, acc.w);
        }
    }
#pragma unroll
    for (int m = kLPR; m < 64; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m, 64);
        acc.y += __shfl_xor(acc.y, m, 64);
        acc.z += __shfl_xor(acc.z, m, 64);
        acc.w += __shfl_xor(acc.w, m, 64);
    }
    if (g == 0 && col_ok)
        *reinterpret_cast<float4 *>(a.y + (b * a.T * a.H + t * a.H + h) * a.d_v + col) = acc;
}

// ------------------------------------------------------------------ update

// One wavefront per (chain, block of kRPI*SPG sorted write events, 128-byte
// row slice); each row group takes SPG consecutive events.  With `rev` the
// chains are taken last to first: the read kernel before it (or the previous
// update) ends on the last chains, whose rows may still sit in the
// memory-side cache (measured: 8.18 -> 8.04 ms write/read per 1.4B-style
// step).  An event whose slot differs from the previous event's starts that
// slot's segment: its group loads the row once, applies the segment's writes
// in time order and stores it once.  Loads of the SPG events are issued
// together.
//
// Lane q of a row group holds event q of the group and the group reads the
// fields with in-group broadcasts, so the events do not take registers in
// every lane (93 VGPRs instead of 125 for a float32 state: five waves per
// SIMD instead of four; write/read 7.81 -> 7.50 ms per 1.4B-style step).
// The group's last segment may go on past the group.  Its next events are
// the next row group's, whose lanes hold their fields and v slices: the
// group takes them from there with cross-lane reads and goes to memory only
// in the wave's last group or for a segment longer than the next group
// (write/read 7.50 -> 7.19 ms; doing the tail inside the per-event loop,
// from memory, forced full waits for every outstanding load).  A bfloat16
// state is held to six waves per SIMD.
template <bool BF16, int SPG, bool SB, bool TAPE = false>
__global__ __launch_bounds__(256, SB ? 6 : 1) void tp_update_kernel(TPArgs a, int ep, int nslice,
                                                                    int nblk, bool rev)
{
    static_assert(!(TAPE && SB), "the tape holds float32 rows");
    using S = StateRow<SB>;
    constexpr int kLPR = S::kLPR, kRPI = 64 / kLPR;
    const int lane = threadIdx.x & 63;
    const int64_t cg = grid_chain();
    const uint32_t u = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (cg >= a.chains || u >= (uint32_t)(nblk * nslice)) return;
    const int slice = (int)(u % (uint32_t)nslice);
    const int blk = (int)(u / (uint32_t)nslice);
    const int64_t chain = rev ? a.chains - 1 - cg : cg;
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int n = ne * a.W;
    const int g = lane / kLPR, q = lane % kLPR;
    const int col = slice * 4 * kLPR + q * 4;
    const bool col_ok = col < a.d_v;
    const int colc = col_ok ? col : 0;
    // chains < 2^32 (the grid's y and z), so 32-bit division
    const int64_t b = (uint32_t)chain / (uint32_t)a.H;
    const int h = (int)(chain - b * a.H);
    const int64_t hd = (int64_t)a.H * a.d_v;
    const int64_t vrow0 = (b * a.T * a.H + h) * a.d_v + colc;
    const rsrc_t Mr = make_rsrc(static_cast<char *>(a.M) + chain * a.N * a.d_v * S::kElem,
                                (uint32_t)(a.N * a.d_v * S::kElem));
    const uint32_t rowb = (uint32_t)a.d_v * S::kElem;
    const TPEntry *se = a.sorted + chain * a.T * a.W + t0 * a.W;
    // TAPE: the epoch-start row of each written slot, stored at the slot of
    // its first write in the epoch ([chain][token][w][column]); the backward
    // recomputes the rows the later writes of the epoch replaced
    float *tape_c = TAPE ? a.tape + (chain * a.T + t0) * a.W * a.d_v + colc : nullptr;
    auto tape_put = [&](const TPEntry &ev, float4 x, bool on) {
        if (TAPE && on)
            *reinterpret_cast<float4 *>(tape_c + ((int64_t)(ev.tw >> 6) * a.W + (ev.tw & 63u)) *
                                                     a.d_v) = x;
    };

    static_assert(SPG <= kLPR, "one event per lane of a row group");
    const int j0 = (blk * kRPI + g) * SPG;
    // lane q < SPG of a row group holds event j0 + q; the group reads the
    // fields back with in-group broadcasts when it needs them
    const TPEntry me = se[(q < SPG && j0 + q < n) ? j0 + q : n - 1];
    const uint32_t next = j0 + SPG < n ? se[j0 + SPG].slot : 0xFFFFFFFFu;
    const uint32_t prev0 = j0 > 0 && j0 - 1 < n ? se[j0 - 1].slot : 0xFFFFFFFFu;
    // bit s of `same`: event s continues the segment of event s - 1 (bit
    // SPG: the event after the group continues the last one's); events are
    // sorted by slot, so a segment is a run of set bits
    uint32_t same = 0u, prev = prev0;
    float4 row[SPG], vv[SPG];
#pragma unroll
    for (int s = 0; s < SPG; s++) {
        const uint32_t sl = group_bcast<kLPR>(me.slot, s);
        const bool in = j0 + s < n;
        same |= (uint32_t)(in & (sl == prev)) << s;
        const bool head = in & (sl != prev);
        row[s] = S::load(Mr, (head & col_ok) ? sl * rowb + col * S::kElem : kOff);
        const uint32_t tw = group_bcast<kLPR>(me.tw, s);
        vv[s] = load_v<BF16>(a.v, vrow0 + (t0 + (tw >> 6)) * hd);
        prev = sl;
    }
    same |= (uint32_t)((j0 + SPG < n) & (next == prev)) << SPG;
    // the group's last segment, when it goes on past the group: finished
    // from memory after the group's other rows are stored
    float4 rt = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t slt = 0u;
    bool tail = false;
#pragma unroll
    for (int s = 0; s < SPG; s++) {
        const bool head = (j0 + s < n) & !((same >> s) & 1u);
        if (TAPE) {
            TPEntry ev;
            ev.tw = group_bcast<kLPR>(me.tw, s);
            tape_put(ev, row[s], head & col_ok);
        }
        float4 r = S::round(fma4(__uint_as_float(group_bcast<kLPR>(__float_as_uint(me.a), s)), row[s],
                                 __uint_as_float(group_bcast<kLPR>(__float_as_uint(me.c), s)), vv[s]));
        // the rest of the segment within the group, in time order
        bool more = true;
#pragma unroll
        for (int s2 = s + 1; s2 < SPG; s2++) {
            more = more & ((same >> s2) & 1u);
            if (more)
                r = S::round(fma4(__uint_as_float(group_bcast<kLPR>(__float_as_uint(me.a), s2)), r,
                                  __uint_as_float(group_bcast<kLPR>(__float_as_uint(me.c), s2)), vv[s2]));
        }
        const uint32_t sl = group_bcast<kLPR>(me.slot, s);
        const bool cont = head & more & ((same >> SPG) & 1u);
        if (cont) {
            rt = r;
            slt = sl;
        }
        tail |= cont;
        S::store(r, Mr, (head & !cont & col_ok) ? sl * rowb + col * S::kElem : kOff);
    }
    // The events just past the group are the next row group's (same wave,
    // same columns, kLPR lanes up): its lanes hold their fields, v rows and
    // which of them continue the segment (leading bits of its `same`).
    int jm = j0 + SPG;  // first event still to apply from memory
    if (__builtin_amdgcn_ballot_w64(tail) != 0ull) {
        const bool inw = g < kRPI - 1;
        const int up = (lane + kLPR) & 63;
        const uint32_t same_nx = (uint32_t)__builtin_amdgcn_ds_bpermute(up * 4, (int)same);
        bool go = tail & inw;
#pragma unroll
        for (int s2 = 0; s2 < SPG; s2++) {
            go = go & ((same_nx >> s2) & 1u);
            if (__builtin_amdgcn_ballot_w64(go) == 0ull) break;
            const int src = ((g + 1) * kLPR + s2) & 63;
            const float a2 = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(me.a)));
            const float c2 = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(me.c)));
            float4 v2;
            v2.x = __int_as_float(__builtin_amdgcn_ds_bpermute(up * 4, __float_as_int(vv[s2].x)));
            v2.y = __int_as_float(__builtin_amdgcn_ds_bpermute(up * 4, __float_as_int(vv[s2].y)));
            v2.z = __int_as_float(__builtin_amdgcn_ds_bpermute(up * 4, __float_as_int(vv[s2].z)));
            v2.w = __int_as_float(__builtin_amdgcn_ds_bpermute(up * 4, __float_as_int(vv[s2].w)));
            if (go) rt = S::round(fma4(a2, rt, c2, v2));
        }
        // the last group of the wave, or a segment that outlasts the next group too
        if (inw) jm = go ? j0 + 2 * SPG : n;
    }
    if (tail) {
        // two events per round trip: both entries load together, then both
        // v slices, so a one-event tail also learns where it ends
        for (int j = jm; j < n; j += 2) {
            const TPEntry f0 = se[j];
            const TPEntry f1 = se[j + 1 < n ? j + 1 : j];
            if (f0.slot != slt) break;
            const bool c1 = (j + 1 < n) & (f1.slot == slt);
            const float4 v0 = load_v<BF16>(a.v, vrow0 + (t0 + (f0.tw >> 6)) * hd);
            const float4 v1 = load_v<BF16>(a.v, vrow0 + (t0 + ((c1 ? f1 : f0).tw >> 6)) * hd);
            rt = S::round(fma4(f0.a, rt, f0.c, v0));
            if (!c1) break;
            rt = S::round(fma4(f1.a, rt, f1.c, v1));
        }
        S::store(rt, Mr, col_ok ? slt * rowb + col * S::kElem : kOff);
    }
}

}  // namespace

#ifndef SDM_TP_EPOCH_LOG2
#define SDM_TP_EPOCH_LOG2 0
#endif

int tp_epoch_len(const Shape &s)
{
    // E <= kMaxEpoch and E*W <= kMaxEpochEvents (replay links pack an event
    // position and a count into 32 bits), and E*W <= 2^SDM_TP_EPOCH_LOG2 * N:
    // longer epochs merge more repeated writes to a slot, but every read
    // then carries more v pairs from in-epoch writes.
    const int64_t cap = SDM_TP_EPOCH_LOG2 >= 0 ? s.N() << SDM_TP_EPOCH_LOG2
                                               : s.N() >> -SDM_TP_EPOCH_LOG2;
    int64_t e = kMaxEpoch;
    while (e > 1 && (e * s.W > kMaxEpochEvents || e * s.W > cap)) e >>= 1;
    if (e > s.T) {
        e = 1;
        while (e < s.T) e <<= 1;
    }
    return (int)e;
}

// v pairs per token: twice the expected number at the end of an epoch
// (R reads, each slot written about E*W/N times per epoch)
static int tp_pair_cap(const Shape &s, int E)
{
    const int64_t m = ((int64_t)E * s.W + s.N() - 1) / s.N();
    const int64_t p = 2 * (int64_t)s.R * (m > 1 ? m : 1);
    return (int)((p + 7) / 8 * 8);
}

size_t tp_workspace_bytes(const Shape &s)
{
    const size_t chains = (size_t)s.B * s.H;
    const size_t ev = chains * (size_t)s.T * s.W;
    const size_t toks = chains * (size_t)s.T;
    const int P = tp_pair_cap(s, tp_epoch_len(s));
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up(ev * sizeof(TPEntry)) + 2 * up(ev * 8) + up(ev * 2) + 2 * up(toks * kMaxK * 4) +
           up(toks * 4) + up(toks * (size_t)P * 8);
}

static TPArgs tp_args(const Shape &s, const uint32_t *rec, void *ws, const void *v, float *y,
                      void *M)
{
    const RecLayout L(s.W, s.R);
    TPArgs a{};
    const size_t chains = (size_t)s.B * s.H;
    const size_t ev = chains * (size_t)s.T * s.W;
    a.E = tp_epoch_len(s);
    a.nepoch = (int)((s.T + a.E - 1) / a.E);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char *p = static_cast<char *>(ws);
    a.sorted = reinterpret_cast<TPEntry *>(p);
    p += up(ev * sizeof(TPEntry));
    a.tmpA = reinterpret_cast<uint64_t *>(p);
    p += up(ev * 8);
    a.tmpB = reinterpret_cast<uint64_t *>(p);
    p += up(ev * 8);
    a.ckey = reinterpret_cast<uint16_t *>(p);
    p += up(ev * 2);
    const size_t toks = chains * (size_t)s.T;
    a.rlink = reinterpret_cast<uint32_t *>(p);
    p += up(toks * kMaxK * 4);
    a.rwt = reinterpret_cast<float *>(p);
    p += up(toks * kMaxK * 4);
    a.npair = reinterpret_cast<uint32_t *>(p);
    p += up(toks * 4);
    a.pairs = reinterpret_cast<uint2 *>(p);
    a.P = tp_pair_cap(s, a.E);
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
    a.chains = (int64_t)chains;
    int bits = 1;
    while ((int64_t(1) << bits) < s.N()) bits++;
    a.passes = (bits + kDigitBits - 1) / kDigitBits;
    a.kshift = bits > 16 ? bits - 16 : 0;
    return a;
}

bool tp_supported(const Shape &s)
{
    // 32-bit buffer offsets within one chain's float32 state (a bfloat16
    // state takes half of that)
    return s.d_v % 4 == 0 && (double)s.N() * s.d_v * 4.0 <= 2147483648.0;
}

hipError_t launch_tp_prepare(const Shape &s, const uint32_t *rec, void *ws, hipStream_t st,
                             int ep0, int ep1, bool link)
{
    TPArgs a = tp_args(s, rec, ws, nullptr, nullptr, nullptr);
    if (ep1 < 0 || ep1 > a.nepoch) ep1 = a.nepoch;
    if (ep0 >= ep1) return hipSuccess;
    a.ep0 = ep0;
    a.nrun = ep1 - ep0;
    const int64_t blocks = a.chains * a.nrun;
    const SortIO io{a.sorted, a.tmpA, a.tmpB, a.ckey};
    hipLaunchKernelGGL(tp_sort_kernel<false>, dim3((unsigned)blocks), dim3(kSortThreads), 0, st, a,
                       io);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !link) return e;
    // sampled coarse keys: at most 32768 of them (64 KiB of LDS)
    const int64_t nmax = (int64_t)a.E * s.W;
    const int stride = nmax > 32768 ? (int)((nmax + 32767) / 32768) : 1;
    // with every write sampled and keys equal to slots, also the tokens (at
    // most 64 KiB in all)
    const int exact = stride == 1 && a.kshift == 0 && nmax <= 16384;
    const size_t lds = (size_t)((nmax + stride - 1) / stride) * sizeof(uint16_t) * (exact ? 2 : 1);
    hipLaunchKernelGGL(tp_link_kernel, dim3((unsigned)blocks), dim3(kSortThreads), lds, st, a,
                       stride, exact);
    return hipGetLastError();
}

template <bool SB>
static hipError_t tp_apply_state(const Shape &s, TPArgs a, bool bf16, hipStream_t st, int ep0,
                                 int ep1)
{
    constexpr int kLPR = StateRow<SB>::kLPR, kRPI = 64 / kLPR;
    const int nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    const int nr = (s.R + kRPI - 1) / kRPI;
    for (int ep = ep0; ep < ep1; ep++) {
        const int64_t t0 = (int64_t)ep * a.E;
        const int ne = (int)((s.T - t0) < a.E ? (s.T - t0) : a.E);
        const dim3 rgrid = chain_grid(a.chains, (int64_t)ne * nslice);
#define SDM_TP_READ(NR_)                                                                          \
    if (nr <= NR_) {                                                                              \
        if (bf16) hipLaunchKernelGGL((tp_read_kernel<NR_, true, SB>), rgrid, dim3(256), 0, st, a, \
                                     ep, nslice);                                                 \
        else hipLaunchKernelGGL((tp_read_kernel<NR_, false, SB>), rgrid, dim3(256), 0, st, a, ep, \
                                nslice);                                                          \
    } else
        SDM_TP_READ(1) SDM_TP_READ(2) SDM_TP_READ(4) SDM_TP_READ(8) SDM_TP_READ(16) {
            return hipErrorInvalidValue;
        }
#undef SDM_TP_READ
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // sorted events per row group (measured at the 1.4B-style layer,
        // write/read: 8 rather than 4, 8.05 -> 7.81 ms, for a float32 state
        // and 5.53 -> 5.23 ms for a bfloat16 state; 16 is slower for both)
        constexpr int SPG = 8;
        const int nblk = (ne * s.W + kRPI * SPG - 1) / (kRPI * SPG);
        const dim3 ugrid = chain_grid(a.chains, (int64_t)nblk * nslice);
        if (bf16)
            hipLaunchKernelGGL((tp_update_kernel<true, SPG, SB>), ugrid, dim3(256), 0, st, a, ep,
                               nslice, nblk, true);
        else
            hipLaunchKernelGGL((tp_update_kernel<false, SPG, SB>), ugrid, dim3(256), 0, st, a, ep,
                               nslice, nblk, true);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tp_forward_tape(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                                  bool bf16, float *M, float *tape, hipStream_t st)
{
    TPArgs a = tp_args(s, rec, ws, v, nullptr, M);
    a.tape = tape;
    // 8 events per row group, as in the forward (backward step 32.43 -> 32.11 ms
    // against 4 at the 1.4B-style layer)
    constexpr int kLPR = StateRow<false>::kLPR, kRPI = 64 / kLPR, SPG = 8;
    const int nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    for (int ep = 0; ep < a.nepoch; ep++) {
        const int64_t t0 = (int64_t)ep * a.E;
        const int ne = (int)((s.T - t0) < a.E ? (s.T - t0) : a.E);
        const int nblk = (ne * s.W + kRPI * SPG - 1) / (kRPI * SPG);
        const dim3 ugrid = chain_grid(a.chains, (int64_t)nblk * nslice);
        const bool rev = ep & 1;  // each launch starts on the chains the previous one ended on
        if (bf16)
            hipLaunchKernelGGL((tp_update_kernel<true, SPG, false, true>), ugrid, dim3(256), 0, st, a,
                               ep, nslice, nblk, rev);
        else
            hipLaunchKernelGGL((tp_update_kernel<false, SPG, false, true>), ugrid, dim3(256), 0, st,
                               a, ep, nslice, nblk, rev);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tp_sort_merged(const Shape &s, const uint32_t *rec, void *ws, TPEntry *out,
                                 uint64_t *tmpA, uint64_t *tmpB, hipStream_t st)
{
    TPArgs a = tp_args(s, rec, ws, nullptr, nullptr, nullptr);
    a.ep0 = 0;
    a.nrun = a.nepoch;
    const SortIO io{out, tmpA, tmpB, nullptr};
    hipLaunchKernelGGL(tp_sort_kernel<true>, dim3((unsigned)(a.chains * a.nrun)),
                       dim3(kSortThreads), 0, st, a, io);
    return hipGetLastError();
}

hipError_t launch_tp_apply(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                           bool bf16, float *y, void *M, bool state_bf16, hipStream_t st, int ep0,
                           int ep1)
{
    TPArgs a = tp_args(s, rec, ws, v, y, M);
    if (ep1 < 0 || ep1 > a.nepoch) ep1 = a.nepoch;
    return state_bf16 ? tp_apply_state<true>(s, a, bf16, st, ep0, ep1)
                      : tp_apply_state<false>(s, a, bf16, st, ep0, ep1);
}

}  // namespace sdm
