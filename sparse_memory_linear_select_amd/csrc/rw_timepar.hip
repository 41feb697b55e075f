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
//            with a bfloat16 or E4M3 state, whose rows are rounded after
//            every write, a read instead gets its in-epoch writes themselves;
//   read     y_t = weighted sum of epoch-start rows and v rows, all gathers
//            independent of each other (narrower states: the epoch-start row
//            with the read's in-epoch writes replayed, rounded as stored);
//   update   the first event of each slot's segment loads the row once,
//            applies all of the segment's writes in time order and stores it
//            once.
//
// Within an epoch everything is parallel; epochs follow each other in stream
// order (read of epoch e, update of e, read of e+1, ...).  Each row value is
// produced by the same float32 operations, in the same order, as in the
// token-serial schedule, so both schedules give identical M; with a float32
// state y agrees to float32 rounding (its terms are grouped differently).
#include "tp_device.h"

#include <cstdlib>

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
    float ssc, sisc;  // E4M3 state: 2^s and 2^-s (the scale of the stored codes)
    float *tape;    // backward's forward pass: [chain][tapeT][W][d_v] epoch-start rows
    int64_t tapeT, tape_t0;  // tokens per chain in the tape, token of its first entry
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
// order.  One read of the records gives the digit histograms of every pass.
// Each scatter tile loads the next tile's items (and, in the last pass, its
// own events' coefficients) before it ranks, so those loads are in flight
// across the tile's barriers; the per-wave digit counts alternate between two
// LDS buffers, the idle one cleared during the scan, so a tile takes two
// barriers.  The last pass writes the 16-byte entries and a
// 16-bit coarse key (slot >> kshift) per entry for the link search.
constexpr int kMaxPasses = (kSlotBits + kDigitBits - 1) / kDigitBits;

template <bool MERGED>
__global__ __launch_bounds__(kSortThreads) void tp_sort_kernel(TPArgs a, SortIO io)
{
    const int ept = MERGED ? a.W + a.R : a.W;  // events per token
    __shared__ uint32_t bins[kMaxPasses][kBuckets];
    __shared__ uint32_t wcnt[2][kWaves][kBuckets];
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
    auto rec_slot = [&](int j) -> uint32_t {  // slot of event j (k >= W: read k - W)
        const int tl = j / ept, k = j - tl * ept;
        const int col = (MERGED && k >= a.W) ? 3 * a.Wp + (k - a.W) : k;
        return recc[(int64_t)tl * a.rec_dwords + col] & kSlotMask;
    };

    // histograms of all digits, four events per thread in flight
    for (int k = tid; k < kMaxPasses * kBuckets; k += kSortThreads) (&bins[0][0])[k] = 0;
    __syncthreads();
    for (int j0 = tid; j0 < n; j0 += 4 * kSortThreads) {
        uint32_t sl[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = j0 + u * kSortThreads;
            sl[u] = j < n ? rec_slot(j) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            if (j0 + u * kSortThreads >= n) break;
            for (int p = 0; p < a.passes; p++)
                atomicAdd(&bins[p][(sl[u] >> (kDigitBits * p)) & (kBuckets - 1)], 1u);
        }
    }
    __syncthreads();
    if (wv == 0) {  // exclusive scan of each pass's buckets, kBuckets/64 per lane
        constexpr int PER = kBuckets / 64;
        for (int p = 0; p < a.passes; p++) {
            uint32_t c[PER], sum = 0;
            for (int k = 0; k < PER; k++) {
                c[k] = bins[p][lane * PER + k];
                sum += c[k];
            }
            uint32_t incl = sum;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = (uint32_t)__shfl_up((int)incl, o, 64);
                if (lane >= o) incl += t;
            }
            uint32_t run = incl - sum;
            for (int k = 0; k < PER; k++) {
                bins[p][lane * PER + k] = run;
                run += c[k];
            }
        }
    }
    __syncthreads();

    for (int p = 0; p < a.passes; p++) {
        const int shift = kDigitBits * p;
        const uint64_t *src = (p & 1) ? io.tmpA + base : io.tmpB + base;  // unused when p == 0
        uint64_t *dst = (p & 1) ? io.tmpB + base : io.tmpA + base;
        const bool last = p == a.passes - 1;
        auto item = [&](int j) -> uint64_t {  // (slot << 32) | event j
            if (p == 0) return ((uint64_t)rec_slot(j) << 32) | (uint32_t)j;
            return src[j];
        };
        uint32_t *pbins = bins[p];
        for (int k = tid; k < kWaves * kBuckets; k += kSortThreads) (&wcnt[0][0][0])[k] = 0;
        __syncthreads();
        // stable scatter, one tile of kSortThreads events at a time
        uint64_t nxt = tid < n ? item(tid) : 0;
        int buf = 0;
        for (int tb = 0; tb < n; tb += kSortThreads) {
            const int j = tb + tid;
            const bool valid = j < n;
            const uint64_t it = nxt;
            if (j + kSortThreads < n) nxt = item(j + kSortThreads);
            // last pass: this event's 16-byte entry, its words loaded now
            TPEntry e;
            if (last && valid) {
                const uint32_t ev = (uint32_t)it;
                const int tl = (int)(ev / (uint32_t)ept), k = (int)(ev - tl * ept);
                const float *rf = reinterpret_cast<const float *>(recc + (int64_t)tl * a.rec_dwords);
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
            }
            const uint32_t dg = (uint32_t)(it >> (32 + shift)) & (kBuckets - 1);
            uint64_t peers = __ballot(valid);  // lanes of this wave with the same digit
            for (int bit = 0; bit < kDigitBits; bit++) {
                const uint64_t m = __ballot((dg >> bit) & 1u);
                peers &= ((dg >> bit) & 1u) ? m : ~m;
            }
            const uint32_t rank = (uint32_t)__popcll(peers & lanes_below);
            // wcnt[buf] is zero: cleared before the pass or during the scan two tiles back
            if (valid && rank == 0) wcnt[buf][wv][dg] = (uint32_t)__popcll(peers);
            __syncthreads();
            for (int d = tid; d < kBuckets; d += kSortThreads) {  // per digit, in wave order
                uint32_t run = pbins[d];
                for (int w = 0; w < kWaves; w++) {
                    const uint32_t c = wcnt[buf][w][d];
                    wcnt[buf][w][d] = run;
                    run += c;
                }
                pbins[d] = run;
            }
            // the other buffer was last read by the previous tile's scatter, before the barrier above
            for (int k = tid; k < kWaves * kBuckets; k += kSortThreads) (&wcnt[buf ^ 1][0][0])[k] = 0;
            __syncthreads();
            if (valid) {
                const uint32_t pos = wcnt[buf][wv][dg] + rank;
                if (!last) {
                    dst[pos] = it;
                } else {
                    io.out[base + pos] = e;
                    if (!MERGED) io.ckey[base + pos] = (uint16_t)(e.slot >> a.kshift);
                }
            }
            buf ^= 1;
        }
        __syncthreads();  // this pass's stores and wcnt reads before the next pass
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
// 64 KiB; with the writes' tokens too, 128 KiB, when every write is sampled
// and keys are slots): a binary search there brackets the slot, a short
// forward scan of the entries finds the exact range.  One wavefront per token: lane r takes
// read r, a prefix sum over the lanes places the pairs.
//
// With `stored` (a bfloat16 or E4M3 state) a read must see the row as the
// state holds it, rounded after every write, which no composed weight can
// give.  There every read keeps weight q, a read that sees in-epoch writes
// gets the link (first write, count) to replay them, and the token's pair
// area holds, per read, the first two of those writes: token, a, c of the
// first at [r], [R + r], [2R + r], of the second at [3R + r], [4R + r],
// [5R + r] (6R dwords <= the 2P dwords of the area, as P >= 3R).
__global__ __launch_bounds__(kSortThreads) void tp_link_kernel(TPArgs a, int stride, int exact,
                                                               int stored, int parts)
{
    extern __shared__ uint16_t ck[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // `parts` workgroups per (chain, epoch), each planning a contiguous range
    // of its tokens
    const int64_t ce = blockIdx.x / parts;
    const int part = (int)(blockIdx.x - ce * parts);
    const int64_t chain = ce / a.nrun;
    const int ep = a.ep0 + (int)(ce - chain * a.nrun);
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const int n = ne * a.W;
    const int ns = (n + stride - 1) / stride;
    const int64_t base = chain * a.T * a.W + t0 * a.W;
    const uint32_t *recc = a.rec + (chain * a.T + t0) * a.rec_dwords;
    const TPEntry *se = a.sorted + base;
    // exact (every write sampled, keys = slots): the token of every sorted
    // write sits in LDS as well, and the searches never touch memory.
    // exact == 2 (the slot table fits too): st[s] = the first sorted write
    // whose slot is >= s, for s in [0, N], so a read's writes are
    // [st[s], st[s + 1]) without a search; otherwise a binary search over the
    // keys in LDS finds the first.
    const bool direct = exact == 2;
    uint16_t *st = ck;
    uint16_t *tk = direct ? ck + (a.N + 1) : ck + ns;
    if (direct) {
        for (int k = tid; k < ns; k += kSortThreads) {
            const int kj = a.ckey[base + k];
            const int kp = k > 0 ? (int)a.ckey[base + k - 1] : -1;
            for (int s2 = kp + 1; s2 <= kj; s2++) st[s2] = (uint16_t)k;
            tk[k] = (uint16_t)(se[k].tw >> 6);
        }
        const int klast = ns > 0 ? (int)a.ckey[base + ns - 1] : -1;
        for (int s2 = klast + 1 + tid; s2 <= (int)a.N; s2 += kSortThreads) st[s2] = (uint16_t)ns;
    } else {
        for (int k = tid; k < ns; k += kSortThreads) {
            ck[k] = a.ckey[base + (int64_t)k * stride];
            if (exact) tk[k] = (uint16_t)(se[k].tw >> 6);
        }
    }
    __syncthreads();
    const int tl0 = (int)((int64_t)ne * part / parts), tl1 = (int)((int64_t)ne * (part + 1) / parts);
    constexpr int kTokStep = kSortThreads / 64;
    const bool real = lane < a.R;
    // the slot and weight of this lane's read, loaded one token ahead
    uint32_t s_nx = 0, q_nx = 0;
    auto load_read = [&](int t) {
        if (t < tl1 && real) {
            const uint32_t *rc = recc + (int64_t)t * a.rec_dwords;
            s_nx = rc[3 * a.Wp + lane] & kSlotMask;
            q_nx = rc[3 * a.Wp + a.Rp + lane];
        }
    };
    load_read(tl0 + (tid >> 6));
    for (int tl = tl0 + (tid >> 6); tl < tl1; tl += kTokStep) {  // wave-uniform token
        const uint32_t s = s_nx;
        const float q = real ? __uint_as_float(q_nx) : 0.0f;
        load_read(tl + kTokStep);
        int j = 0, cnt = 0;
        if (real && direct) {
            j = st[s];
            const int je = st[s + 1];
            int l2 = j;  // past the writes of s at tokens <= tl
            while (l2 < je && (int)tk[l2] <= tl) l2++;
            cnt = l2 - j;
        } else if (real) {
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
        const int64_t ct = chain * a.T + t0 + tl;
        if (stored) {  // wave-uniform
            a.rwt[ct * kMaxK + lane] = q;
            // j < n <= kMaxEpochEvents and cnt <= E < 2^kCntBits
            a.rlink[ct * kMaxK + lane] = cnt > 0 ? (((uint32_t)j << kCntBits) | cnt) : 0u;
            if (cnt > 0) {
                uint32_t *fw = reinterpret_cast<uint32_t *>(a.pairs + ct * a.P);
                const TPEntry e = se[j];
                fw[lane] = e.tw >> 6;
                fw[a.R + lane] = __float_as_uint(e.a);
                fw[2 * a.R + lane] = __float_as_uint(e.c);
                if (cnt > 1) {
                    const TPEntry e2 = se[j + 1];
                    fw[3 * a.R + lane] = e2.tw >> 6;
                    fw[4 * a.R + lane] = __float_as_uint(e2.a);
                    fw[5 * a.R + lane] = __float_as_uint(e2.c);
                }
            }
            if (lane == 0) a.npair[ct] = 0u;
            continue;
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

// Float32 state.  One wavefront per (chain, token of the epoch, 256-byte row
// slice).  With the read plan, y_t = sum_r w_r row_r + sum_j u_j v_(t_j): the
// 4 row groups take their NR reads at once (epoch-start rows), then the
// token's v pairs kPairBatch per group at a time.  Every load depends only on
// the plan, so all of them can be in flight together; reads that overflowed
// the plan replay their writes from the sorted events.
constexpr int kPairBatch = 4;   // v pairs per row group in flight, after the first ones
constexpr int kFirstPairs = 1;  // v pairs per row group loaded with the plan (0 - 3: 1 fastest)

template <int NR, bool BF16>
__global__ __launch_bounds__(256) void tp_read_kernel(TPArgs a, int ep, int nslice)
{
    using S = StateRow<kStateF32>;  // float32 state (narrower states: tp_read_stored_kernel)
    const S st(0.f, 0.f);
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

    // The plan: the pair count, the token's first pairs (the pair area is
    // always there; entries past the count are masked below) and, in lane q
    // of row group g, the slot word and weight of reference g*NR + q (q < NR;
    // the group reads them back with in-group broadcasts).  None of these
    // loads depends on another, so they take one round trip; the row and v
    // gathers then depend only on them and take one more.
    const uint32_t npw_v = a.npair[ct];
    uint2 pr0[kFirstPairs];
#pragma unroll
    for (int u = 0; u < kFirstPairs; u++) {
        const int j = u * kRPI + g;
        pr0[u] = j < a.P ? pp[j] : make_uint2(0u, 0u);
    }
    const bool mine = (q < NR) & (g * NR + q < a.R);
    const uint32_t sl_mine = mine ? rc[3 * a.Wp + g * NR + q] : 0u;
    const float wr_mine = mine ? a.rwt[ct * kMaxK + g * NR + q] : 0.0f;
    const uint32_t npw = __builtin_amdgcn_readfirstlane(npw_v);
    const int np = (int)(npw & ~kReplayFlag);
    // v rows of the first pairs (a pair past the count: weight 0, token 0)
    float4 vv0[kFirstPairs];
#pragma unroll
    for (int u = 0; u < kFirstPairs; u++) {
        if (u * kRPI + g >= np) pr0[u] = make_uint2(0u, 0u);
        vv0[u] = load_v<BF16>(a.v, vrow0 + (t0 + pr0[u].x) * hd);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!(npw & kReplayFlag)) {
        // every row gather at once, then the weighted sum
        typename S::Raw row[NR];
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const uint32_t sl = group_bcast<kLPR>(sl_mine, i);
            const bool ok = col_ok & (g * NR + i < a.R);
            row[i] = st.load_raw(Mr, ok ? (sl & kSlotMask) * rowb + col * S::kElem : kOff);
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            // masked references have weight 0 and a zero row
            const float4 rv = st.widen(row[i]);
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
            float4 rv = st.load(Mr, ok ? (sl & kSlotMask) * rowb + col * S::kElem : kOff);
            // links exist only for the R real references; zero unless the plan overflowed
            const uint32_t l = (g * NR + i < a.R) ? lkp[i] : 0u;
            const int first = (int)(l >> kCntBits), cnt = (int)(l & ((1u << kCntBits) - 1u));
            for (int k = 0; k < cnt; k++) {  // writes of this slot earlier in the epoch
                const TPEntry e = se[first + k];
                const float4 vv = load_v<BF16>(a.v, vrow0 + (t0 + (e.tw >> 6)) * hd);
                rv = st.round(fma4(e.a, rv, e.c, vv));
            }
            const float wr = __uint_as_float(group_bcast<kLPR>(__float_as_uint(wr_mine), i));
            acc.x = fmaf(wr, rv.x, acc.x);
            acc.y = fmaf(wr, rv.y, acc.y);
            acc.z = fmaf(wr, rv.z, acc.z);
            acc.w = fmaf(wr, rv.w, acc.w);
        }
    }
#pragma unroll
    for (int u = 0; u < kFirstPairs; u++) {
        const float wgt = __uint_as_float(pr0[u].y);
        acc.x = fmaf(wgt, vv0[u].x, acc.x);
        acc.y = fmaf(wgt, vv0[u].y, acc.y);
        acc.z = fmaf(wgt, vv0[u].z, acc.z);
        acc.w = fmaf(wgt, vv0[u].w, acc.w);
    }
    // the rest of the pairs (tokens with many in-epoch writes before them)
    for (int j0 = kRPI * kFirstPairs; j0 < np; j0 += kRPI * kPairBatch) {
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

// Read with a bfloat16 or E4M3 state.  The state holds every written row
// rounded, so a read of a slot written earlier in the epoch (at a token <=
// its own) must see the row after each of those writes, rounded: it replays
// them on the epoch-start row with the update kernel's own operations,
// st.round(a*row + c*v) in time order.
//
// The R reads of a (chain, token of the epoch, 128-byte row slice) unit are
// split over WPU wavefronts (a power of two; a unit's waves share a
// workgroup), kStoredNR reads per row group: lane q < kStoredNR of a group
// holds read q's plan -- slot word, weight q, link (first write, count) and
// the first two in-epoch writes' token, a and c.  Every gather that depends only
// on the plan -- the epoch-start rows and the v slices of the first two
// writes -- is issued at once; a third or later write comes from the sorted
// events, one round trip for all of the wave's reads per write.  Each wave
// sums its reads in read order, and the unit's first wave adds the partial
// sums of the others in wave order (LDS), so y sums the R rows in one fixed
// order whichever reads saw in-epoch writes: it does not depend on where
// epochs start.
// Reads per row group, and whether the second write's v is gathered with
// the rows.  Measured at the 1.4B-style layer with a bfloat16 state
// (write/read): 4 reads with the second write 5.67 ms (62 VGPRs, eight waves
// per SIMD), 4 without it 5.97, 8 with it 6.00 (115 VGPRs, four waves), 8
// without it 6.04.
constexpr int kStoredNR = 4;
constexpr bool kSecondWithPlan = true;

// Waves per (chain, token, slice) unit: enough for R reads, a power of two.
template <int ST>
constexpr int stored_waves_per_unit(int R)
{
    const int per_wave = kStoredNR * (64 / StateRow<ST>::kLPR);
    const int w = (R + per_wave - 1) / per_wave;
    return w <= 1 ? 1 : (w <= 2 ? 2 : (w <= 4 ? 4 : 8));
}
static_assert(kStoredNR * 2 * 8 >= kMaxK, "8 waves of 2 row groups hold every read");

template <bool BF16, int ST, int WPU>
__global__ __launch_bounds__(64 * (WPU > 4 ? WPU : 4)) void tp_read_stored_kernel(TPArgs a, int ep,
                                                                                  int nslice)
{
    using S = StateRow<ST>;
    constexpr int kLPR = S::kLPR, kRPI = 64 / kLPR, NR = kStoredNR;
    constexpr int kWG = WPU > 4 ? WPU : 4;  // waves per workgroup
    static_assert(NR <= kLPR && kWG % WPU == 0, "one read per lane; a unit's waves in a workgroup");
    __shared__ float4 part[kWG][kLPR];  // partial sums of the waves (column quads of the slice)
    const S st(a.ssc, a.sisc);
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t chain = grid_chain();
    const int64_t t0 = (int64_t)ep * a.E;
    const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);
    const uint32_t wid = blockIdx.x * (uint32_t)kWG + (uint32_t)wv;  // wave of this chain
    const uint32_t u = wid / WPU;                          // its unit
    const int w = (int)(wid % WPU);                        // its part of the unit's reads
    const bool active = chain < a.chains && u < (uint32_t)(ne * nslice);  // wave-uniform
    const int slice = (int)(u % (uint32_t)nslice);
    const int tl = active ? (int)(u / (uint32_t)nslice) : 0;
    const int64_t t = t0 + tl;
    const int64_t ct = (active ? chain : 0) * a.T + t;
    const int g = lane / kLPR, q = lane % kLPR;
    const int col = slice * 4 * kLPR + q * 4;
    const bool col_ok = active & (col < a.d_v);
    const int colc = col_ok ? col : 0;
    // chains < 2^32 (the grid's y and z), so 32-bit division
    const int64_t b = (uint32_t)chain / (uint32_t)a.H;
    const int h = (int)(chain - b * a.H);
    const int64_t hd = (int64_t)a.H * a.d_v;
    const int64_t vrow0 = (b * a.T * a.H + h) * a.d_v + colc;  // v of token 0 of the chain
    const rsrc_t Mr = make_rsrc(static_cast<char *>(a.M) + (active ? chain : 0) * a.N * a.d_v * S::kElem,
                                (uint32_t)(a.N * a.d_v * S::kElem));
    const uint32_t rowb = (uint32_t)a.d_v * S::kElem;
    const uint32_t *rc = a.rec + ct * a.rec_dwords;
    const TPEntry *se = a.sorted + (active ? chain : 0) * a.T * a.W + t0 * a.W;
    const uint32_t *fw = reinterpret_cast<const uint32_t *>(a.pairs + ct * a.P);

    // this lane's read (lane q < NR of group g): w*kRPI*NR + g*NR + q
    const int r0 = (w * kRPI + g) * NR;
    const int r = r0 + q;
    const bool mine = active & (q < NR) & (r < a.R);
    const uint32_t sl_mine = mine ? rc[3 * a.Wp + r] : 0u;
    const float wr_mine = mine ? a.rwt[ct * kMaxK + r] : 0.0f;
    const uint32_t lk_mine = mine ? a.rlink[ct * kMaxK + r] : 0u;
    // the first two writes' fields: loaded with the rest of the plan (the
    // token's pair area is always there; the fields are used only where the
    // link count says the writes exist)
    const int rr = mine ? r : 0;
    const uint32_t t1m = fw[rr], a1m = fw[a.R + rr], c1m = fw[2 * a.R + rr];
    const uint32_t t2m = fw[3 * a.R + rr], a2m = fw[4 * a.R + rr], c2m = fw[5 * a.R + rr];

    // every gather the plan decides: rows, and v of the first two writes
    typename S::Raw row[NR];
    float4 v1[NR], v2[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const uint32_t sl = group_bcast<kLPR>(sl_mine, i);
        const bool ok = col_ok & (r0 + i < a.R);
        row[i] = st.load_raw(Mr, ok ? (sl & kSlotMask) * rowb + col * S::kElem : kOff);
    }
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const int cnt = (int)(group_bcast<kLPR>(lk_mine, i) & ((1u << kCntBits) - 1u));
        const uint32_t t1 = group_bcast<kLPR>(t1m, i), t2 = group_bcast<kLPR>(t2m, i);
        v1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        v2[i] = v1[i];
        if (cnt > 0) v1[i] = load_v<BF16>(a.v, vrow0 + (t0 + t1) * hd);
        if (kSecondWithPlan && cnt > 1) v2[i] = load_v<BF16>(a.v, vrow0 + (t0 + t2) * hd);
    }
    float4 rv[NR];
    int cnt[NR], first[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const uint32_t lk = group_bcast<kLPR>(lk_mine, i);
        cnt[i] = (int)(lk & ((1u << kCntBits) - 1u));
        first[i] = (int)(lk >> kCntBits);
        rv[i] = st.widen(row[i]);
        if (cnt[i] > 0)
            rv[i] = st.round(fma4(__uint_as_float(group_bcast<kLPR>(a1m, i)), rv[i],
                                  __uint_as_float(group_bcast<kLPR>(c1m, i)), v1[i]));
        if (kSecondWithPlan && cnt[i] > 1)
            rv[i] = st.round(fma4(__uint_as_float(group_bcast<kLPR>(a2m, i)), rv[i],
                                  __uint_as_float(group_bcast<kLPR>(c2m, i)), v2[i]));
    }
    if constexpr (!kSecondWithPlan) {  // second writes: one more round trip
        bool more = false;
#pragma unroll
        for (int i = 0; i < NR; i++) more |= cnt[i] > 1;
        if (__ballot(more) != 0ull) {
#pragma unroll
            for (int i = 0; i < NR; i++) {
                const uint32_t t2 = group_bcast<kLPR>(t2m, i);
                if (cnt[i] > 1) v2[i] = load_v<BF16>(a.v, vrow0 + (t0 + t2) * hd);
            }
#pragma unroll
            for (int i = 0; i < NR; i++)
                if (cnt[i] > 1)
                    rv[i] = st.round(fma4(__uint_as_float(group_bcast<kLPR>(a2m, i)), rv[i],
                                          __uint_as_float(group_bcast<kLPR>(c2m, i)), v2[i]));
        }
    }
    // third and later in-epoch writes (rare): one round trip per write level
    for (int k = 2;; k++) {
        bool more = false;
#pragma unroll
        for (int i = 0; i < NR; i++) more |= k < cnt[i];
        if (__ballot(more) == 0ull) break;
        TPEntry e[NR];
#pragma unroll
        for (int i = 0; i < NR; i++)
            if (k < cnt[i]) e[i] = se[first[i] + k];
#pragma unroll
        for (int i = 0; i < NR; i++) {
            if (k < cnt[i]) {
                const float4 vk = load_v<BF16>(a.v, vrow0 + (t0 + (e[i].tw >> 6)) * hd);
                rv[i] = st.round(fma4(e[i].a, rv[i], e[i].c, vk));
            }
        }
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NR; i++) {
        // masked references have weight 0 and a zero row
        const float wr = __uint_as_float(group_bcast<kLPR>(__float_as_uint(wr_mine), i));
        acc.x = fmaf(wr, rv[i].x, acc.x);
        acc.y = fmaf(wr, rv[i].y, acc.y);
        acc.z = fmaf(wr, rv[i].z, acc.z);
        acc.w = fmaf(wr, rv[i].w, acc.w);
    }
#pragma unroll
    for (int m = kLPR; m < 64; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m, 64);
        acc.y += __shfl_xor(acc.y, m, 64);
        acc.z += __shfl_xor(acc.z, m, 64);
        acc.w += __shfl_xor(acc.w, m, 64);
    }
    if constexpr (WPU > 1) {
        if (g == 0) part[wv][q] = acc;
        __syncthreads();
        if (w != 0) return;
#pragma unroll
        for (int k = 1; k < WPU; k++) {
            const float4 p = part[wv + k][q];
            acc.x += p.x;
            acc.y += p.y;
            acc.z += p.z;
            acc.w += p.w;
        }
    }
    if (g == 0 && col_ok)
        *reinterpret_cast<float4 *>(a.y + (b * a.T * a.H + t * a.H + h) * a.d_v + col) = acc;
}

// ------------------------------------------------------------------ update

// A row group's SPG sorted events (event s in lane s of the group; the row
// of a segment's first event from row_at(s), the v slices from v_at(s))
// applied in one pass, in time order: a segment starts from its loaded row at its first
// event, every event applies row <- round(a*row + c*v) once, and the row is
// stored after the segment's last event in the group.  The group's leading
// events may continue a segment of the group before, whose group applies
// them: they are skipped.  A segment that goes on past the group (bit SPG of
// `same`) is not stored but left in rt / slt with tail set.  on_head(s, h)
// sees each event with h = whether it starts a segment.  A narrow state
// takes one pass (one fma and one rounding per event; applying each segment
// from its head over the rest of the group cost up to SPG*(SPG+1)/2, and the
// roundings made that the larger part of a narrow-state write: bfloat16
// write/read 5.64 -> 4.88 ms at the 1.4B-style layer with the fused kernel);
// a float32 state keeps the per-head form, whose segments are independent
// chains (the one pass: 6.74 -> 6.82 ms).
template <int kLPR, int SPG, class S, class RowAt, class VAt, class OnHead>
__device__ __forceinline__ void apply_group(const S &st, const TPEntry &me, uint32_t same, int j0,
                                            int n, RowAt row_at, VAt v_at, rsrc_t Mr,
                                            uint32_t rowb, int col, bool col_ok, float4 &rt,
                                            uint32_t &slt, bool &tail, OnHead on_head)
{
    if constexpr (S::kElem == 4) {
        tail = false;
#pragma unroll
        for (int s = 0; s < SPG; s++) {
            const bool head = (j0 + s < n) & !((same >> s) & 1u);
            on_head(s, head);
            float4 r = fma4(__uint_as_float(group_bcast<kLPR>(__float_as_uint(me.a), s)), row_at(s),
                            __uint_as_float(group_bcast<kLPR>(__float_as_uint(me.c), s)), v_at(s));
            bool more = true;  // the rest of the segment within the group, in time order
#pragma unroll
            for (int s2 = s + 1; s2 < SPG; s2++) {
                more = more & ((same >> s2) & 1u);
                if (more)
                    r = fma4(__uint_as_float(group_bcast<kLPR>(__float_as_uint(me.a), s2)), r,
                             __uint_as_float(group_bcast<kLPR>(__float_as_uint(me.c), s2)), v_at(s2));
            }
            const uint32_t sl = group_bcast<kLPR>(me.slot, s);
            const bool cont = head & more & ((same >> SPG) & 1u);
            if (cont) {
                rt = r;
                slt = sl;
            }
            tail |= cont;
            st.store(r, Mr, (head & !cont & col_ok) ? sl * rowb + col * S::kElem : kOff);
        }
        return;
    }
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    bool act = false;  // inside a segment this group applies
#pragma unroll
    for (int s = 0; s < SPG; s++) {
        const bool cont = (same >> s) & 1u;  // set only for events in range
        const bool head = (j0 + s < n) & !cont;
        on_head(s, head);
        act = head | (act & cont);
        if (head) r = row_at(s);
        if (act)
            r = st.round(fma4(__uint_as_float(group_bcast<kLPR>(__float_as_uint(me.a), s)), r,
                              __uint_as_float(group_bcast<kLPR>(__float_as_uint(me.c), s)), v_at(s)));
        const uint32_t sl = group_bcast<kLPR>(me.slot, s);
        const bool nxt = (same >> (s + 1)) & 1u;  // event s + 1 (bit SPG: past the group) continues
        if (s == SPG - 1) {
            tail = act & nxt;
            if (tail) {
                rt = r;
                slt = sl;
            }
        }
        st.store(r, Mr, (act & !nxt & col_ok) ? sl * rowb + col * S::kElem : kOff);
    }
}

// One wavefront per (chain, block of kRPI*SPG sorted write events, row
// slice); each row group takes SPG consecutive events.  With `rev` the
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
// or E4M3 state is held to six waves per SIMD, a float32 state (no tape) to
// five, which the compiler otherwise misses by a few registers.
template <bool BF16, int SPG, int ST, bool TAPE = false>
__global__ __launch_bounds__(256, ST != kStateF32 ? 6 : (TAPE ? 1 : 5)) void tp_update_kernel(TPArgs a, int ep,
                                                                                 int nslice,
                                                                                 int nblk, bool rev)
{
    static_assert(!(TAPE && ST != kStateF32), "the tape holds float32 rows");
    using S = StateRow<ST>;
    const S st(a.ssc, a.sisc);
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
    float *tape_c =
        TAPE ? a.tape + (chain * a.tapeT + (t0 - a.tape_t0)) * a.W * a.d_v + colc : nullptr;
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
        row[s] = st.load(Mr, (head & col_ok) ? sl * rowb + col * S::kElem : kOff);
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
    apply_group<kLPR, SPG>(st, me, same, j0, n, [&](int s) { return row[s]; },
                           [&](int s) { return vv[s]; }, Mr, rowb, col, col_ok, rt, slt, tail,
                           [&](int s, bool head) {
                               if (TAPE) {
                                   TPEntry ev;
                                   ev.tw = group_bcast<kLPR>(me.tw, s);
                                   tape_put(ev, row[s], head & col_ok);
                               }
                           });
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
            if (go) rt = st.round(fma4(a2, rt, c2, v2));
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
            rt = st.round(fma4(f0.a, rt, f0.c, v0));
            if (!c1) break;
            rt = st.round(fma4(f1.a, rt, f1.c, v1));
        }
        st.store(rt, Mr, col_ok ? slt * rowb + col * S::kElem : kOff);
    }
}

// ------------------------------------------------------------------ fused apply

// Bfloat16 or E4M3 state, epochs of at most kFuseMaxE tokens.  One workgroup
// of kFuseWaves waves per (chain, 64-column slice) takes every epoch of the
// call: it stages the epoch's v rows (its columns, float32) in LDS, does the
// epoch's reads, then its writes, then the next epoch, with a barrier between
// the phases.  No other workgroup touches its columns of the chain's state,
// so a barrier orders everything the phases share, and the v slices that the
// replayed and applied writes need come from LDS rather than from the cache
// hierarchy.  Each row and each y element is computed with the operations of
// tp_read_stored_kernel and tp_update_kernel in their order (the same
// butterfly and wave order for y), so the results are bit-identical to
// theirs; the per-epoch launches remain for epochs too long to stage and for
// shapes with fewer units than compute units.
constexpr int kFuseWaves = 16;
constexpr int kFuseLPR = 16;     // lanes per row group: 64 columns per slice
constexpr int kFuseMaxE = 256;   // tokens of v in LDS: kFuseMaxE * 256 bytes

template <bool BF16, int ST>
__global__ __launch_bounds__(64 * kFuseWaves) void tp_fused_stored_kernel(TPArgs a, int ep0,
                                                                          int ep1)
{
    using S = StateRow<ST>;
    constexpr int kLPR = kFuseLPR, kRPI = 64 / kLPR, NR = kStoredNR, SPG = 16;
    // tp_read_stored_kernel's order: a wave there adds its row groups' sums
    // of NR reads by a butterfly, and its unit adds the waves' sums in order;
    // here a row group takes kLPR reads, i.e. kOldPerGroup of those waves
    constexpr int kOldRPI = 64 / S::kLPR;
    constexpr int kPerOld = NR * kOldRPI;
    constexpr int kOldPerGroup = kLPR / kPerOld;
    constexpr int kMaxOld = kRPI * kOldPerGroup;
    static_assert(kLPR % kPerOld == 0 && kRPI * kLPR >= kMaxK && (kOldRPI == 2 || kOldRPI == 4),
                  "a row group holds whole waves of the per-epoch read");
    static_assert(SPG <= kLPR, "one event per lane of a row group");
    __shared__ float4 vs[kFuseMaxE * kLPR];
    const S st(a.ssc, a.sisc);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // unit = slice * chains + chain: with chains a multiple of 8, the slices
    // of a chain share an XCD (workgroups go to XCDs round-robin) and its
    // plan is fetched into one L2
    const int64_t chain = (int64_t)(blockIdx.x % (uint32_t)a.chains);
    const int slice = (int)(blockIdx.x / (uint32_t)a.chains);
    // Per-lane values are derived from the lane number anew in every
    // iteration of the loops below: the empty asm hides that the number is
    // the same each time, so they are recomputed in a few instructions
    // rather than kept live across the whole kernel (which spilled them).
    auto lane_ids = [&](int &g, int &q, int &col, bool &col_ok) {
        int ln = (int)(threadIdx.x & 63);
        asm volatile("" : "+v"(ln));
        g = ln / kLPR;
        q = ln % kLPR;
        col = slice * 4 * kLPR + q * 4;
        col_ok = col < a.d_v;
    };
    // chains < 2^32, so 32-bit division
    const int64_t b = (uint32_t)chain / (uint32_t)a.H;
    const int h = (int)(chain - b * a.H);
    const int64_t hd = (int64_t)a.H * a.d_v;
    const int64_t vrow0 = (b * a.T * a.H + h) * a.d_v;  // v of token 0 of the chain, column 0
    const rsrc_t Mr = make_rsrc(static_cast<char *>(a.M) + chain * a.N * a.d_v * S::kElem,
                                (uint32_t)(a.N * a.d_v * S::kElem));
    const uint32_t rowb = (uint32_t)a.d_v * S::kElem;
    const int wpu_old = stored_waves_per_unit<ST>(a.R);

    for (int ep = ep0; ep < ep1; ep++) {
        const int64_t t0 = (int64_t)ep * a.E;
        const int ne = (int)((a.T - t0) < a.E ? (a.T - t0) : a.E);  // <= kFuseMaxE (host check)
        const int n = ne * a.W;
        const TPEntry *se = a.sorted + chain * a.T * a.W + t0 * a.W;
        {  // the epoch's v rows: every load issued, then the LDS stores
            constexpr int kStage = kFuseMaxE * kLPR / (64 * kFuseWaves);
            float4 vt[kStage];
#pragma unroll
            for (int u = 0; u < kStage; u++) {
                const int i = (int)threadIdx.x + u * 64 * kFuseWaves;
                const int c = slice * 4 * kLPR + (i % kLPR) * 4;
                vt[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (i < ne * kLPR && c < a.d_v) vt[u] = load_v<BF16>(a.v, vrow0 + (t0 + i / kLPR) * hd + c);
            }
#pragma unroll
            for (int u = 0; u < kStage; u++) {
                const int i = (int)threadIdx.x + u * 64 * kFuseWaves;
                if (i < ne * kLPR) vs[i] = vt[u];
            }
        }
        __syncthreads();

        // reads: one token per wave at a time; lane q of row group g holds
        // the plan of read g*kLPR + q
        // a token's plan, loaded one token ahead (the rows of a token wait
        // only for its own plan, which arrived during the previous token)
        struct Plan {
            uint32_t sl, wr, lk, t12, a1, c1, a2, c2;  // t12: the two writes' tokens (< 2^16)
        };
        auto load_plan = [&](int tl) {
            int g, q, col;
            bool col_ok;
            lane_ids(g, q, col, col_ok);
            const int64_t ct = chain * a.T + t0 + tl;
            const uint32_t *rc = a.rec + ct * a.rec_dwords;
            const uint32_t *fw = reinterpret_cast<const uint32_t *>(a.pairs + ct * a.P);
            const bool mine = g * kLPR + q < a.R;
            const int rr = mine ? g * kLPR + q : 0;
            Plan p;
            p.sl = mine ? rc[3 * a.Wp + rr] : 0u;
            p.wr = mine ? __float_as_uint(a.rwt[ct * kMaxK + rr]) : 0u;
            p.lk = mine ? a.rlink[ct * kMaxK + rr] : 0u;
            p.t12 = (fw[rr] & 0xFFFFu) | (fw[3 * a.R + rr] << 16);
            p.a1 = fw[a.R + rr];
            p.c1 = fw[2 * a.R + rr];
            p.a2 = fw[4 * a.R + rr];
            p.c2 = fw[5 * a.R + rr];
            return p;
        };
        Plan pnext{};
        if (wv < ne) pnext = load_plan(wv);
        for (int tl = wv; tl < ne; tl += kFuseWaves) {
            int g, q, col;
            bool col_ok;
            lane_ids(g, q, col, col_ok);
            const int64_t t = t0 + tl;
            const int r0 = g * kLPR;
            const Plan pl0 = pnext;
            const uint32_t sl_mine = pl0.sl, lk_mine = pl0.lk;
            const float wr_mine = __uint_as_float(pl0.wr);
            const uint32_t t12m = pl0.t12, a1m = pl0.a1, c1m = pl0.c1;
            const uint32_t a2m = pl0.a2, c2m = pl0.c2;
            typename S::Raw row[kLPR];
#pragma unroll
            for (int i = 0; i < kLPR; i++) {
                const uint32_t sl = group_bcast<kLPR>(sl_mine, i);
                const bool ok = col_ok & (r0 + i < a.R);
                row[i] = st.load_raw(Mr, ok ? (sl & kSlotMask) * rowb + col * S::kElem : kOff);
            }
            if (tl + kFuseWaves < ne) pnext = load_plan(tl + kFuseWaves);
            // sums of NR reads (the per-epoch read's row groups), folded as
            // soon as they are complete, in its butterfly's order: with 4 row
            // groups there a wave sum is (p0 + p1) + (p2 + p3), with 2 p0 + p1
            float4 sw[kOldPerGroup], pl = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int bq = 0; bq < kLPR / NR; bq++) {
                float4 rv[NR];
                int cnt[NR], first[NR];
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    const int k = bq * NR + i;
                    const uint32_t lk = group_bcast<kLPR>(lk_mine, k);
                    cnt[i] = (int)(lk & ((1u << kCntBits) - 1u));
                    first[i] = (int)(lk >> kCntBits);
                    rv[i] = st.widen(row[k]);
                    if (cnt[i] > 0)
                        rv[i] = st.round(fma4(__uint_as_float(group_bcast<kLPR>(a1m, k)), rv[i],
                                              __uint_as_float(group_bcast<kLPR>(c1m, k)),
                                              vs[(cnt[i] > 0 ? group_bcast<kLPR>(t12m, k) & 0xFFFFu : 0u) * kLPR + q]));
                    if (cnt[i] > 1)
                        rv[i] = st.round(fma4(__uint_as_float(group_bcast<kLPR>(a2m, k)), rv[i],
                                              __uint_as_float(group_bcast<kLPR>(c2m, k)),
                                              vs[(cnt[i] > 1 ? group_bcast<kLPR>(t12m, k) >> 16 : 0u) * kLPR + q]));
                }
                // third and later in-epoch writes (rare): read by read, one
                // event at a time, which keeps the registers of the common
                // path free
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    for (int k = 2; k < cnt[i]; k++) {
                        const TPEntry e = se[first[i] + k];
                        rv[i] = st.round(fma4(e.a, rv[i], e.c, vs[(e.tw >> 6) * kLPR + q]));
                    }
                }
                float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    // masked references have weight 0 and a zero row
                    const float wr = __uint_as_float(group_bcast<kLPR>(__float_as_uint(wr_mine), bq * NR + i));
                    acc.x = fmaf(wr, rv[i].x, acc.x);
                    acc.y = fmaf(wr, rv[i].y, acc.y);
                    acc.z = fmaf(wr, rv[i].z, acc.z);
                    acc.w = fmaf(wr, rv[i].w, acc.w);
                }
                if (bq % 2 == 0) {
                    pl = acc;
                } else {
                    const float4 pr = make_float4(pl.x + acc.x, pl.y + acc.y, pl.z + acc.z, pl.w + acc.w);
                    if constexpr (kOldRPI == 2) {
                        sw[bq / 2] = pr;
                    } else if (bq % 4 == 1) {
                        sw[bq / 4] = pr;
                    } else {
                        const float4 x = sw[bq / 4];
                        sw[bq / 4] = make_float4(x.x + pr.x, x.y + pr.y, x.z + pr.z, x.w + pr.w);
                    }
                }
            }
            // its unit's sum of the waves, in wave order (wave o of row group g
            // is wave g*kOldPerGroup + o there)
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < kMaxOld; w++) {
                const int src = (w / kOldPerGroup) * kLPR + q;
                float4 p;
                p.x = __shfl(sw[w % kOldPerGroup].x, src, 64);
                p.y = __shfl(sw[w % kOldPerGroup].y, src, 64);
                p.z = __shfl(sw[w % kOldPerGroup].z, src, 64);
                p.w = __shfl(sw[w % kOldPerGroup].w, src, 64);
                if (w == 0) {
                    y = p;
                } else if (w < wpu_old) {
                    y.x += p.x;
                    y.y += p.y;
                    y.z += p.z;
                    y.w += p.w;
                }
            }
            if (g == 0 && col_ok)
                *reinterpret_cast<float4 *>(a.y + (b * a.T * a.H + t * a.H + h) * a.d_v + col) = y;
        }
        __syncthreads();

        // writes: tp_update_kernel's blocks of kRPI*SPG sorted events
        const int nblk = (n + kRPI * SPG - 1) / (kRPI * SPG);
        // a block's events, loaded one block ahead
        struct Block {
            TPEntry me;
            uint32_t next, prev0;
        };
        auto load_block = [&](int blk) {
            int g, q, col;
            bool col_ok;
            lane_ids(g, q, col, col_ok);
            const int j0 = (blk * kRPI + g) * SPG;
            Block k;
            k.me = se[(q < SPG && j0 + q < n) ? j0 + q : n - 1];
            k.next = j0 + SPG < n ? se[j0 + SPG].slot : 0xFFFFFFFFu;
            k.prev0 = j0 > 0 && j0 - 1 < n ? se[j0 - 1].slot : 0xFFFFFFFFu;
            return k;
        };
        Block bnext{};
        if (wv < nblk) bnext = load_block(wv);
        for (int blk = wv; blk < nblk; blk += kFuseWaves) {
            int g, q, col;
            bool col_ok;
            lane_ids(g, q, col, col_ok);
            const int lane = g * kLPR + q;
            const int j0 = (blk * kRPI + g) * SPG;
            const Block cur = bnext;
            const TPEntry me = cur.me;
            const uint32_t next = cur.next;
            uint32_t same = 0u, prev = cur.prev0;
            typename S::Raw row[SPG];  // in the state's width until used
#pragma unroll
            for (int s = 0; s < SPG; s++) {
                const uint32_t sl = group_bcast<kLPR>(me.slot, s);
                const bool in = j0 + s < n;
                same |= (uint32_t)(in & (sl == prev)) << s;
                const bool head = in & (sl != prev);
                row[s] = st.load_raw(Mr, (head & col_ok) ? sl * rowb + col * S::kElem : kOff);
                prev = sl;
            }
            if (blk + kFuseWaves < nblk) bnext = load_block(blk + kFuseWaves);
            same |= (uint32_t)((j0 + SPG < n) & (next == prev)) << SPG;
            float4 rt = make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t slt = 0u;
            bool tail = false;
            apply_group<kLPR, SPG>(
                st, me, same, j0, n, [&](int s) { return st.widen(row[s]); },
                [&](int s) { return vs[(group_bcast<kLPR>(me.tw, s) >> 6) * kLPR + q]; }, Mr, rowb,
                col, col_ok, rt, slt, tail, [](int, bool) {});
            // the segment goes on into the next row group (its lanes hold the
            // fields and v slices), then from memory
            int jm = j0 + SPG;
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
                    const uint32_t tw2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)me.tw);
                    const float4 v2 = vs[(tw2 >> 6) * kLPR + q];
                    if (go) rt = st.round(fma4(a2, rt, c2, v2));
                }
                if (inw) jm = go ? j0 + 2 * SPG : n;
            }
            if (tail) {
                for (int j = jm; j < n; j += 2) {
                    const TPEntry f0 = se[j];
                    const TPEntry f1 = se[j + 1 < n ? j + 1 : j];
                    if (f0.slot != slt) break;
                    const bool c1 = (j + 1 < n) & (f1.slot == slt);
                    const float4 v0 = vs[(f0.tw >> 6) * kLPR + q];
                    const float4 v1 = vs[((c1 ? f1 : f0).tw >> 6) * kLPR + q];
                    rt = st.round(fma4(f0.a, rt, f0.c, v0));
                    if (!c1) break;
                    rt = st.round(fma4(f1.a, rt, f1.c, v1));
                }
                st.store(rt, Mr, col_ok ? slt * rowb + col * S::kElem : kOff);
            }
        }
        __syncthreads();
    }
}

}  // namespace

// Whether the (chain, 64-column slice) units of tp_fused_stored_kernel give
// every one of `cus` compute units one workgroup in every round (one fits a
// compute unit at a time): a whole number of rounds, or enough of them that
// a partial last one costs little.
static bool fused_units_fill(const Shape &s, int64_t cus)
{
    const int64_t units = (int64_t)s.B * s.H * ((s.d_v + 4 * kFuseLPR - 1) / (4 * kFuseLPR));
    return units >= cus && (units % cus == 0 || units >= 8 * cus);
}

// The compute units the epoch rule assumes: an MI355X's 256.  A fixed figure
// keeps the epoch length, and with it every workspace size, a pure function
// of the shape (any epoch length gives correct results; the launches
// themselves use the device's own count).
constexpr int64_t kEpochRuleCUs = 256;

// Tokens per epoch with E*W <= cap: the largest power of two <= kMaxEpoch
// with E*W <= kMaxEpochEvents (replay links pack an event position and a
// count into 32 bits) and E*W <= cap.
static int64_t epoch_for_cap(const Shape &s, int64_t cap)
{
    int64_t e = kMaxEpoch;
    while (e > 1 && (e * s.W > kMaxEpochEvents || e * s.W > cap)) e >>= 1;
    return e;
}

int tp_epoch_len(const Shape &s, bool stored)
{
    // Longer epochs merge more repeated writes to a slot and take fewer
    // launches, but every read then carries more v pairs from in-epoch
    // writes, and the sort (one workgroup per (chain, epoch)) has fewer
    // workgroups.  A float32 state takes E*W <= 2N where chains x epochs
    // still give a quarter of the compute units a sort workgroup, else
    // E*W <= N (1.4B-style layer, write/read and step: E*W = N 6.74 / 7.77
    // ms, 2N 6.06 / 7.30, 4N 6.63 / 8.52; 8B-style layer 27.52 / 32.53 at
    // N, 25.45 / 31.66 at 2N; larger state, 8 chains and 64 sort
    // workgroups at 2N: 13.66 / 15.92 at N, 12.62 / 15.38 at 2N with the
    // plan split over 4 workgroups per (chain, epoch), 12.85 / 16.40 without
    // that split).  A bfloat16 or E4M3 state keeps E*W <= N: each of its
    // reads replays its in-epoch writes.
    int64_t e = epoch_for_cap(s, 2 * s.N());
    const int64_t groups = (int64_t)s.B * s.H * ((s.T + e - 1) / e);
    if (stored || 4 * groups < kEpochRuleCUs) e = epoch_for_cap(s, s.N());
    // A bfloat16 or E4M3 state: every read sees the stored rows, so neither
    // y nor M depends on where epochs start.  Where the fused kernel's units
    // fill the GPU, epochs short enough for it to stage their v rows let it
    // take the whole apply in one launch (8B-style layer: bf16 write/read
    // 21.85 -> 21.42 ms, E4M3 20.10 -> 16.11 ms against 1024-token epochs in
    // per-epoch launches).
    if (stored && e > kFuseMaxE && fused_units_fill(s, kEpochRuleCUs)) e = kFuseMaxE;
    if (e > s.T) {
        e = 1;
        while (e < s.T) e <<= 1;
    }
    return (int)e;
}

// v pairs per token: twice the expected number at the end of an epoch
// (R reads, each slot written about E*W/N times per epoch), and at least
// 3R, which the stored-value plan needs (two writes per read, 3 dwords each)
static int tp_pair_cap(const Shape &s, int E)
{
    const int64_t m = ((int64_t)E * s.W + s.N() - 1) / s.N();
    int64_t p = 2 * (int64_t)s.R * (m > 1 ? m : 1);
    if (p < 3 * (int64_t)s.R) p = 3 * (int64_t)s.R;
    return (int)((p + 7) / 8 * 8);
}

size_t tp_workspace_bytes(const Shape &s, bool stored)
{
    const size_t chains = (size_t)s.B * s.H;
    const size_t ev = chains * (size_t)s.T * s.W;
    const size_t toks = chains * (size_t)s.T;
    const int P = tp_pair_cap(s, tp_epoch_len(s, stored));
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up(ev * sizeof(TPEntry)) + 2 * up(ev * 8) + up(ev * 2) + 2 * up(toks * kMaxK * 4) +
           up(toks * 4) + up(toks * (size_t)P * 8);
}

static TPArgs tp_args(const Shape &s, const uint32_t *rec, void *ws, const void *v, float *y,
                      void *M, bool stored = false)
{
    const RecLayout L(s.W, s.R);
    TPArgs a{};
    const size_t chains = (size_t)s.B * s.H;
    const size_t ev = chains * (size_t)s.T * s.W;
    a.E = tp_epoch_len(s, stored);
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
                             int ep0, int ep1, bool link, bool stored)
{
    TPArgs a = tp_args(s, rec, ws, nullptr, nullptr, nullptr, stored);
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
    // most 128 KiB in all: 32 768 writes, the 1.4B-style layer's 512-token
    // epochs; step 7.29 -> 7.21 ms against the sampled search there)
    int exact = stride == 1 && a.kshift == 0 && nmax <= 32768;
    size_t lds = (size_t)((nmax + stride - 1) / stride) * sizeof(uint16_t) * (exact ? 2 : 1);
    // and the table of each slot's first write where it fits with the tokens
    // (N + 1 + E W 16-bit words: 96 KiB at the 1.4B-style layer)
    if (exact && (a.N + 1 + nmax) * (int64_t)sizeof(uint16_t) <= 131072) {
        exact = 2;
        lds = (size_t)(a.N + 1 + nmax) * sizeof(uint16_t);
    }
    // fewer (chain, epoch) pairs than compute units: split each one's tokens
    // over up to 4 workgroups (each loads the epoch's keys itself; 8B-style
    // layer, 128 pairs in 2 parts: step 31.6 -> 30.8 ms)
    const int64_t cus = compute_units();
    int parts = 1;
    while (parts < 4 && blocks * parts * 2 <= cus) parts *= 2;
    hipLaunchKernelGGL(tp_link_kernel, dim3((unsigned)(blocks * parts)), dim3(kSortThreads), lds,
                       st, a, stride, exact, stored ? 1 : 0, parts);
    return hipGetLastError();
}

// Whether a narrow-state apply takes tp_fused_stored_kernel: its epochs must
// fit the LDS buffer; then the environment variable SDM_TP_FUSED=0 keeps the
// per-epoch launches and SDM_TP_FUSED=1 takes the fused kernel (the results
// are bit-identical either way), and otherwise it is taken when its units
// fill the GPU (fused_units_fill).
static bool use_fused(const TPArgs &a, const Shape &s)
{
    if (a.E > kFuseMaxE) return false;
    const char *env = getenv("SDM_TP_FUSED");
    if (env && env[0] == '0') return false;
    if (env && env[0] == '1') return true;
    return fused_units_fill(s, compute_units());
}

template <int ST>
static hipError_t tp_apply_state(const Shape &s, TPArgs a, bool bf16, hipStream_t st, int ep0,
                                 int ep1)
{
    if constexpr (ST != kStateF32) {
        if (use_fused(a, s)) {
            const int64_t units = a.chains * ((s.d_v + 4 * kFuseLPR - 1) / (4 * kFuseLPR));
            if (units >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
            if (ep0 >= ep1) return hipSuccess;
            if (bf16)
                hipLaunchKernelGGL((tp_fused_stored_kernel<true, ST>), dim3((unsigned)units),
                                   dim3(64 * kFuseWaves), 0, st, a, ep0, ep1);
            else
                hipLaunchKernelGGL((tp_fused_stored_kernel<false, ST>), dim3((unsigned)units),
                                   dim3(64 * kFuseWaves), 0, st, a, ep0, ep1);
            return hipGetLastError();
        }
    }
    constexpr int kLPR = StateRow<ST>::kLPR, kRPI = 64 / kLPR;
    const int nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    const int nr = (s.R + kRPI - 1) / kRPI;
    for (int ep = ep0; ep < ep1; ep++) {
        const int64_t t0 = (int64_t)ep * a.E;
        const int ne = (int)((s.T - t0) < a.E ? (s.T - t0) : a.E);
        const dim3 rgrid = chain_grid(a.chains, (int64_t)ne * nslice);
        if constexpr (ST != kStateF32) {  // stored-value reads (rows rounded after every write)
            const int wpu = stored_waves_per_unit<ST>(s.R);
            const int wg = wpu > 4 ? wpu : 4;  // waves per workgroup
            const int64_t waves = (int64_t)ne * nslice * wpu;
            dim3 sgrid = chain_grid(a.chains, waves);
            sgrid.x = (unsigned)((waves + wg - 1) / wg);
#define SDM_TP_READ(W_)                                                                           \
    if (wpu == W_) {                                                                              \
        if (bf16) hipLaunchKernelGGL((tp_read_stored_kernel<true, ST, W_>), sgrid, dim3(64 * wg), \
                                     0, st, a, ep, nslice);                                       \
        else hipLaunchKernelGGL((tp_read_stored_kernel<false, ST, W_>), sgrid, dim3(64 * wg), 0,  \
                                st, a, ep, nslice);                                               \
    } else
            SDM_TP_READ(1) SDM_TP_READ(2) SDM_TP_READ(4) SDM_TP_READ(8) {
                return hipErrorInvalidValue;
            }
#undef SDM_TP_READ
        } else {
#define SDM_TP_READ(NR_)                                                                          \
    if (nr <= NR_) {                                                                              \
        if (bf16) hipLaunchKernelGGL((tp_read_kernel<NR_, true>), rgrid, dim3(256), 0, st, a, ep, \
                                     nslice);                                                     \
        else hipLaunchKernelGGL((tp_read_kernel<NR_, false>), rgrid, dim3(256), 0, st, a, ep,     \
                                nslice);                                                          \
    } else
            SDM_TP_READ(1) SDM_TP_READ(2) SDM_TP_READ(4) SDM_TP_READ(8) SDM_TP_READ(16) {
                return hipErrorInvalidValue;
            }
#undef SDM_TP_READ
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // sorted events per row group (measured at the 1.4B-style layer,
        // write/read: 8 rather than 4, 8.05 -> 7.81 ms, for a float32 state
        // and 5.53 -> 5.23 ms for a bfloat16 state; 16 is slower for both)
        constexpr int SPG = 8;
        const int nblk = (ne * s.W + kRPI * SPG - 1) / (kRPI * SPG);
        const dim3 ugrid = chain_grid(a.chains, (int64_t)nblk * nslice);
        if (bf16)
            hipLaunchKernelGGL((tp_update_kernel<true, SPG, ST>), ugrid, dim3(256), 0, st, a, ep,
                               nslice, nblk, true);
        else
            hipLaunchKernelGGL((tp_update_kernel<false, SPG, ST>), ugrid, dim3(256), 0, st, a, ep,
                               nslice, nblk, true);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tp_forward_tape(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                                  bool bf16, float *M, float *tape, int64_t tapeT,
                                  int64_t tape_t0, int ep0, int ep1, hipStream_t st)
{
    TPArgs a = tp_args(s, rec, ws, v, nullptr, M);
    a.tape = tape;
    a.tapeT = tapeT;
    a.tape_t0 = tape_t0;
    if (ep1 < 0 || ep1 > a.nepoch) ep1 = a.nepoch;
    // 8 events per row group, as in the forward (backward step 32.43 -> 32.11 ms
    // against 4 at the 1.4B-style layer)
    constexpr int kLPR = StateRow<kStateF32>::kLPR, kRPI = 64 / kLPR, SPG = 8;
    const int nslice = (s.d_v + 4 * kLPR - 1) / (4 * kLPR);
    for (int ep = ep0; ep < ep1; ep++) {
        const int64_t t0 = (int64_t)ep * a.E;
        const int ne = (int)((s.T - t0) < a.E ? (s.T - t0) : a.E);
        const int nblk = (ne * s.W + kRPI * SPG - 1) / (kRPI * SPG);
        const dim3 ugrid = chain_grid(a.chains, (int64_t)nblk * nslice);
        const bool rev = ep & 1;  // each launch starts on the chains the previous one ended on
        if (tape) {
            if (bf16)
                hipLaunchKernelGGL((tp_update_kernel<true, SPG, kStateF32, true>), ugrid, dim3(256),
                                   0, st, a, ep, nslice, nblk, rev);
            else
                hipLaunchKernelGGL((tp_update_kernel<false, SPG, kStateF32, true>), ugrid, dim3(256),
                                   0, st, a, ep, nslice, nblk, rev);
        } else {  // state only (the checkpoint pass)
            if (bf16)
                hipLaunchKernelGGL((tp_update_kernel<true, SPG, kStateF32>), ugrid, dim3(256), 0, st,
                                   a, ep, nslice, nblk, rev);
            else
                hipLaunchKernelGGL((tp_update_kernel<false, SPG, kStateF32>), ugrid, dim3(256), 0, st,
                                   a, ep, nslice, nblk, rev);
        }
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
                           bool bf16, float *y, void *M, StateFmt fmt, hipStream_t st, int ep0,
                           int ep1)
{
    TPArgs a = tp_args(s, rec, ws, v, y, M, fmt.type != kStateF32);
    a.ssc = ldexpf(1.0f, fmt.scale_log2);
    a.sisc = ldexpf(1.0f, -fmt.scale_log2);
    if (ep1 < 0 || ep1 > a.nepoch) ep1 = a.nepoch;
    switch (fmt.type) {
        case kStateBF16: return tp_apply_state<kStateBF16>(s, a, bf16, st, ep0, ep1);
        case kStateFP8: return tp_apply_state<kStateFP8>(s, a, bf16, st, ep0, ep1);
        default: return tp_apply_state<kStateF32>(s, a, bf16, st, ep0, ep1);
    }
}

}  // namespace sdm
