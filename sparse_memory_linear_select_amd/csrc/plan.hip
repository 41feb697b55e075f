// Forwarding planner for the token-serial write/read kernel.
//
// The serial kernel prefetches the rows of token t while earlier tokens are
// still being written, so a prefetched row is stale when one of the previous
// (depth-1) tokens wrote the same slot; a read row must also see the write of
// its own token (the read follows the write, explainer "Sparse Delta Memory：
// 通过稀疏性扩展线性 RNN 的状态容量", §3.1 step 3).  For every slot reference of
// every token this pass finds the most recent such write (token distance d,
// position w' in that token's write list) and stores it in the slot word, so
// the serial kernel can take the row from its on-chip copy instead.
//
// One workgroup per (chain, block of 64 tokens): the write lists of the block
// and of the depth-1 tokens before it are sorted by slot in LDS (one
// wavefront-wide bitonic sort per token), then every reference is resolved by
// binary search, newest token first.
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int kTB = 64;  // tokens per workgroup

struct PlanArgs {
    uint32_t *rec;
    int64_t T;
    int W, R, Wp, rec_dwords, depth;
    int64_t nblk;
};

__global__ __launch_bounds__(256) void plan_kernel(PlanArgs a)
{
    __shared__ uint32_t keys[kTB + kMaxDepth - 1][64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t chain = blockIdx.x / a.nblk;
    const int64_t t0 = (blockIdx.x - chain * a.nblk) * kTB;
    const int64_t first = t0 - (a.depth - 1);  // token of keys[0]
    const int64_t tlo = first < 0 ? 0 : first;
    const int64_t thi = t0 + kTB < a.T ? t0 + kTB : a.T;
    uint32_t *base = a.rec + chain * a.T * a.rec_dwords;

    // sorted (slot << 6 | w) of each write list
    for (int64_t tt = tlo + wv; tt < thi; tt += 4) {
        const uint32_t *r = base + tt * a.rec_dwords;
        uint32_t key = lane < a.W ? (((r[lane] & kSlotMask) << 6) | (uint32_t)lane) : 0xFFFFFFFFu;
#pragma unroll
        for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
            for (int j = kk >> 1; j > 0; j >>= 1) {
                const uint32_t o = (uint32_t)__shfl_xor((int)key, j, 64);
                const bool keep_min = ((lane & j) == 0) == ((lane & kk) == 0);
                key = keep_min ? (key < o ? key : o) : (key > o ? key : o);
            }
        }
        keys[tt - first][lane] = key;
    }
    __syncthreads();

    const int nref = a.W + a.R;
    const int64_t total = (thi - t0) * nref;
    for (int64_t i = threadIdx.x; i < total; i += blockDim.x) {
        const int64_t tt = t0 + i / nref;
        const int e = (int)(i % nref);
        uint32_t *word = base + tt * a.rec_dwords + (e < a.W ? e : 3 * a.Wp + (e - a.W));
        const uint32_t slot = *word & kSlotMask;
        const uint32_t target = slot << 6;
        for (int d = e < a.W ? 1 : 0; d < a.depth; d++) {
            const int64_t tp = tt - d;
            if (tp < 0) break;
            const uint32_t *k = keys[tp - first];
            int lo = 0, hi = a.W;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (k[mid] < target) lo = mid + 1;
                else hi = mid;
            }
            if (lo < a.W && (k[lo] >> 6) == slot) {
                *word = slot | kFwdValid | ((uint32_t)d << kFwdDShift) |
                        ((k[lo] & kFwdWMask) << kFwdWShift);
                break;
            }
        }
    }
}

}  // namespace

hipError_t launch_plan(const Shape &s, uint32_t *rec, int depth, hipStream_t st)
{
    if (depth <= 0) return hipSuccess;
    const RecLayout L(s.W, s.R);
    PlanArgs a{};
    a.rec = rec;
    a.T = s.T;
    a.W = s.W;
    a.R = s.R;
    a.Wp = L.Wp;
    a.rec_dwords = L.dwords();
    a.depth = depth;
    a.nblk = (s.T + kTB - 1) / kTB;
    const int64_t blocks = (int64_t)s.B * s.H * a.nblk;
    hipLaunchKernelGGL(plan_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace sdm
