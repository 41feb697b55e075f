// Broadcast of the shared initial state: M[b] <- M_0 for every sequence b
// (explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量", §3.1,
// learned initial state; "Technical Summary: Sparse Delta Memory (SDM)",
// Learned Initial State).  Streaming copy: each float4 of M_0 is read once
// and written B times.  A bfloat16 state receives M_0 rounded to nearest,
// ties to even; an E4M3 state the codes of M_0 * 2^-s (nearest, ties to
// even, saturating).
#include "sdm_internal.h"

namespace sdm {
namespace {

__global__ __launch_bounds__(256) void init_kernel(const float *__restrict__ M0,
                                                   float *__restrict__ M, int64_t n, int B)
{
    const int64_t n4 = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4 *src = reinterpret_cast<const float4 *>(M0);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 x = src[i];
        for (int b = 0; b < B; b++) reinterpret_cast<float4 *>(M + (int64_t)b * n)[i] = x;
    }
    // tail (n not a multiple of 4)
    for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = M0[i];
        for (int b = 0; b < B; b++) M[(int64_t)b * n + i] = x;
    }
}

// Per-sequence copy when the slab size breaks float4 alignment of M[b].
__global__ __launch_bounds__(256) void init_kernel_scalar(const float *__restrict__ M0,
                                                          float *__restrict__ M, int64_t n, int B)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = M0[i];
        for (int b = 0; b < B; b++) M[(int64_t)b * n + i] = x;
    }
}

// bfloat16 state: n is a multiple of 4 (d_v % 4 == 0), so every 4 values of
// a sequence's slab are 8-byte aligned.
__global__ __launch_bounds__(256) void init_kernel_bf16(const float *__restrict__ M0,
                                                        uint2 *__restrict__ M, int64_t n, int B)
{
    const int64_t n4 = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4 *src = reinterpret_cast<const float4 *>(M0);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 x = src[i];
        const uint2 u = make_uint2(bf16_pack2(x.x, x.y), bf16_pack2(x.z, x.w));
        for (int b = 0; b < B; b++) M[(int64_t)b * n4 + i] = u;
    }
}

// E4M3 state: 4 codes per 32-bit word (n is a multiple of 4).
__global__ __launch_bounds__(256) void init_kernel_fp8(const float *__restrict__ M0,
                                                       uint32_t *__restrict__ M, int64_t n, int B,
                                                       float isc)
{
    const int64_t n4 = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4 *src = reinterpret_cast<const float4 *>(M0);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 x = src[i];
        const uint32_t u = e4m3_pack4(x.x * isc, x.y * isc, x.z * isc, x.w * isc);
        for (int b = 0; b < B; b++) M[(int64_t)b * n4 + i] = u;
    }
}

}  // namespace

hipError_t launch_init(const Shape &s, const float *M0, void *Mv, StateFmt fmt, hipStream_t st)
{
    const int64_t n = (int64_t)s.H * s.N() * s.d_v;  // values per sequence
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (fmt.type == kStateFP8) {
        if (n & 3) return hipErrorInvalidValue;  // callers check d_v % 4 == 0
        hipLaunchKernelGGL(init_kernel_fp8, dim3((unsigned)blocks), dim3(256), 0, st, M0,
                           static_cast<uint32_t *>(Mv), n, s.B, ldexpf(1.0f, -fmt.scale_log2));
        return hipGetLastError();
    }
    if (fmt.type == kStateBF16) {
        if (n & 3) return hipErrorInvalidValue;  // callers check d_v % 4 == 0
        hipLaunchKernelGGL(init_kernel_bf16, dim3((unsigned)blocks), dim3(256), 0, st, M0,
                           static_cast<uint2 *>(Mv), n, s.B);
        return hipGetLastError();
    }
    float *M = static_cast<float *>(Mv);
    if ((n & 3) == 0)
        hipLaunchKernelGGL(init_kernel, dim3((unsigned)blocks), dim3(256), 0, st, M0, M, n, s.B);
    else
        hipLaunchKernelGGL(init_kernel_scalar, dim3((unsigned)blocks), dim3(256), 0, st, M0, M, n,
                           s.B);
    return hipGetLastError();
}

}  // namespace sdm
