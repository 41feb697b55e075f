// Device helpers shared by the time-parallel forward and backward kernels:
// raw buffer loads/stores (out-of-range offsets load zero and drop stores),
// the affine row update, v loads, the float32/bfloat16 state row access and
// in-group lane broadcasts, and the chain grid of per-chain launches.
// Included by one translation unit each, so the
// definitions stay internal to it.
#pragma once

#include "sdm_internal.h"

namespace sdm {
namespace {

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOff = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;

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
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, (int)off, 0, 0);
}

__device__ __forceinline__ float4 fma4(float a, float4 x, float c, float4 v)
{
    return make_float4(fmaf(a, x.x, c * v.x), fmaf(a, x.y, c * v.y), fmaf(a, x.z, c * v.z),
                       fmaf(a, x.w, c * v.w));
}

// Row storage of the state.  Every lane holds 4 columns of a row; a row
// slice is the 128 bytes that LPR lanes cover (the fabric's request size).
//   float32 state: 8 lanes x 16 bytes;
//   bfloat16 state: 16 lanes x 8 bytes, widened exactly on load, rounded to
//   nearest-even after every write (the value the state holds).
template <bool SB>
struct StateRow;

template <>
struct StateRow<false> {
    static constexpr int kLPR = 8;
    static constexpr uint32_t kElem = 4;
    using Raw = float4;
    static __device__ __forceinline__ Raw load_raw(rsrc_t r, uint32_t off) { return buf_load4(r, off); }
    static __device__ __forceinline__ float4 widen(Raw x) { return x; }
    static __device__ __forceinline__ float4 load(rsrc_t r, uint32_t off) { return buf_load4(r, off); }
    static __device__ __forceinline__ void store(float4 v, rsrc_t r, uint32_t off)
    {
        buf_store4(v, r, off);
    }
    static __device__ __forceinline__ float4 round(float4 v) { return v; }
};

template <>
struct StateRow<true> {
    static constexpr int kLPR = 16;
    static constexpr uint32_t kElem = 2;
    using Raw = uint2;  // 4 bfloat16 values
    static __device__ __forceinline__ Raw load_raw(rsrc_t r, uint32_t off)
    {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        return make_uint2(u[0], u[1]);
    }
    static __device__ __forceinline__ float4 widen(Raw u)
    {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
    static __device__ __forceinline__ float4 load(rsrc_t r, uint32_t off) { return widen(load_raw(r, off)); }
    static __device__ __forceinline__ void store(float4 v, rsrc_t r, uint32_t off)
    {
        __attribute__((ext_vector_type(2))) unsigned u;
        u[0] = bf16_bits(v.x) | (bf16_bits(v.y) << 16);
        u[1] = bf16_bits(v.z) | (bf16_bits(v.w) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(u, r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ float4 round(float4 v)
    {
        return make_float4(__uint_as_float(bf16_bits(v.x) << 16), __uint_as_float(bf16_bits(v.y) << 16),
                           __uint_as_float(bf16_bits(v.z) << 16), __uint_as_float(bf16_bits(v.w) << 16));
    }
};

template <bool BF16>
__device__ __forceinline__ float4 load_v(const void *v, int64_t off)
{
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(v) + off);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
        return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(v) + off);
    }
}

// Value of x in lane (lane & ~(LPR - 1)) | i, i.e. lane i of this lane's
// group of LPR lanes (LPR = 8 or 16): ds_swizzle in bit mode acts within 32
// lanes as lane' = (lane & and_mask) | or_mask.
// (i is a constant once the callers' loops are unrolled, so the switch folds
// to one instruction; the swizzle pattern must be an immediate.)
template <int LPR>
__device__ __forceinline__ uint32_t group_bcast(uint32_t x, int i)
{
    static_assert(LPR == 8 || LPR == 16, "row groups of 8 or 16 lanes");
    constexpr int kAnd = 0x1F & ~(LPR - 1);
    const int v = (int)x;
    switch (i) {
#define SDM_SWZ(I) \
    case I: return (uint32_t)__builtin_amdgcn_ds_swizzle(v, kAnd | ((I) << 5));
        SDM_SWZ(0) SDM_SWZ(1) SDM_SWZ(2) SDM_SWZ(3) SDM_SWZ(4) SDM_SWZ(5) SDM_SWZ(6) SDM_SWZ(7)
        SDM_SWZ(8) SDM_SWZ(9) SDM_SWZ(10) SDM_SWZ(11) SDM_SWZ(12) SDM_SWZ(13) SDM_SWZ(14)
        SDM_SWZ(15)
#undef SDM_SWZ
    }
    return 0u;
}

template <int K, typename T>
__device__ __forceinline__ void load_k(const T *p, T (&out)[K])
{
    if constexpr (K % 4 == 0 && sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < K; i += 4) {
            const uint4 x = *reinterpret_cast<const uint4 *>(p + i);
            out[i] = __builtin_bit_cast(T, x.x);
            out[i + 1] = __builtin_bit_cast(T, x.y);
            out[i + 2] = __builtin_bit_cast(T, x.z);
            out[i + 3] = __builtin_bit_cast(T, x.w);
        }
    } else if constexpr (K == 2 && sizeof(T) == 4) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        out[0] = __builtin_bit_cast(T, x.x);
        out[1] = __builtin_bit_cast(T, x.y);
    } else {
#pragma unroll
        for (int i = 0; i < K; i++) out[i] = p[i];
    }
}

// Grid of a launch over every chain: x covers one chain's waves (four to a
// workgroup), y and z the chains (y at most 65535), so the kernels split
// their wave index with 32-bit arithmetic.
static dim3 chain_grid(int64_t chains, int64_t waves_per_chain)
{
    const unsigned gy = (unsigned)(chains < 65535 ? chains : 65535);
    return dim3((unsigned)((waves_per_chain + 3) / 4), gy, (unsigned)((chains + gy - 1) / gy));
}

__device__ __forceinline__ int64_t grid_chain()
{
    return (int64_t)blockIdx.y + (int64_t)blockIdx.z * gridDim.y;
}

}  // namespace
}  // namespace sdm
