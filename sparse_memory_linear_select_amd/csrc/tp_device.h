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
// slice is what the kLPR lanes of a row group cover:
//   float32 state: 16 lanes x 16 bytes = 256 bytes (against 8 lanes and
//   128 bytes: write/read 7.12 -> 6.82 ms at the 1.4B-style layer, 29.36 ->
//   27.56 ms at the 8B-style layer; 32 lanes for the update alone, 6.88);
//   bfloat16 state: 16 lanes x 8 bytes = 128 bytes (32 lanes: slower, 5.65
//   -> 5.76 ms), widened exactly on load, rounded to nearest-even after
//   every write (the value the state holds);
//   E4M3 state: 32 lanes x 4 bytes = 128 bytes, codes of the values scaled by 2^-s,
//   decoded exactly and scaled by 2^s on load, encoded (nearest-even,
//   saturating) after every write.
// An object carries the scale (sc = 2^s, isc = 2^-s; unused by the other
// types): `const S st(sc, isc);` then st.load(...), st.store(...).
template <int ST>
struct StateRow;

template <>
struct StateRow<kStateF32> {
    static constexpr int kLPR = 16;
    static constexpr uint32_t kElem = 4;
    using Raw = float4;
    __device__ StateRow(float, float) {}
    __device__ __forceinline__ Raw load_raw(rsrc_t r, uint32_t off) const { return buf_load4(r, off); }
    __device__ __forceinline__ float4 widen(Raw x) const { return x; }
    __device__ __forceinline__ float4 load(rsrc_t r, uint32_t off) const { return buf_load4(r, off); }
    __device__ __forceinline__ void store(float4 v, rsrc_t r, uint32_t off) const
    {
        buf_store4(v, r, off);
    }
    __device__ __forceinline__ float4 round(float4 v) const { return v; }
    __device__ __forceinline__ Raw pack(float4 v) const { return v; }
};

template <>
struct StateRow<kStateBF16> {
    static constexpr int kLPR = 16;
    static constexpr uint32_t kElem = 2;
    using Raw = uint2;  // 4 bfloat16 values
    __device__ StateRow(float, float) {}
    __device__ __forceinline__ Raw load_raw(rsrc_t r, uint32_t off) const
    {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        return make_uint2(u[0], u[1]);
    }
    __device__ __forceinline__ float4 widen(Raw u) const
    {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
    __device__ __forceinline__ float4 load(rsrc_t r, uint32_t off) const { return widen(load_raw(r, off)); }
    // the 4 values rounded to bfloat16, packed
    __device__ __forceinline__ Raw pack(float4 v) const
    {
        return make_uint2(bf16_pack2(v.x, v.y), bf16_pack2(v.z, v.w));
    }
    __device__ __forceinline__ void store(float4 v, rsrc_t r, uint32_t off) const
    {
        const uint2 p = pack(v);
        __attribute__((ext_vector_type(2))) unsigned u;
        u[0] = p.x;
        u[1] = p.y;
        __builtin_amdgcn_raw_buffer_store_b64(u, r, (int)off, 0, 0);
    }
    __device__ __forceinline__ float4 round(float4 v) const
    {
        return widen(pack(v));
    }
};

template <>
struct StateRow<kStateFP8> {
    static constexpr int kLPR = 32;
    static constexpr uint32_t kElem = 1;
    using Raw = uint32_t;  // 4 E4M3 codes, column k in byte k
    float sc, isc;
    __device__ StateRow(float sc_, float isc_) : sc(sc_), isc(isc_) {}
    __device__ __forceinline__ Raw load_raw(rsrc_t r, uint32_t off) const
    {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    __device__ __forceinline__ float4 widen(Raw u) const
    {
        return make_float4(e4m3_value<0>(u) * sc, e4m3_value<1>(u) * sc, e4m3_value<2>(u) * sc,
                           e4m3_value<3>(u) * sc);
    }
    __device__ __forceinline__ float4 load(rsrc_t r, uint32_t off) const { return widen(load_raw(r, off)); }
    __device__ __forceinline__ Raw pack(float4 v) const
    {
        return e4m3_pack4(v.x * isc, v.y * isc, v.z * isc, v.w * isc);
    }
    __device__ __forceinline__ void store(float4 v, rsrc_t r, uint32_t off) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(pack(v), r, (int)off, 0, 0);
    }
    __device__ __forceinline__ float4 round(float4 v) const { return widen(pack(v)); }
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
// group of LPR lanes.  LPR = 16: the DPP row broadcast row_newbcast:i, a VALU
// move within each row of 16 lanes (the LDS pipe stays free; every caller
// runs it where a row's lanes are all active or all inactive, since a DPP
// read of an inactive lane is undefined).  LPR = 8 or 32: ds_swizzle in bit
// mode, which acts within 32 lanes as lane' = (lane & and_mask) | or_mask.
// (i is a constant once the callers' loops are unrolled, so the switch folds
// to one instruction; the DPP control and the swizzle pattern are immediates.)
template <int LPR>
__device__ __forceinline__ uint32_t group_bcast(uint32_t x, int i)
{
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row groups of 8, 16 or 32 lanes");
    const int v = (int)x;
    if constexpr (LPR == 16) {
        switch (i) {
#define SDM_NBC(I) \
    case I: return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x150 + (I), 0xF, 0xF, false);
            SDM_NBC(0) SDM_NBC(1) SDM_NBC(2) SDM_NBC(3) SDM_NBC(4) SDM_NBC(5) SDM_NBC(6) SDM_NBC(7)
            SDM_NBC(8) SDM_NBC(9) SDM_NBC(10) SDM_NBC(11) SDM_NBC(12) SDM_NBC(13) SDM_NBC(14)
            SDM_NBC(15)
#undef SDM_NBC
        }
        return 0u;
    }
    constexpr int kAnd = 0x1F & ~(LPR - 1);
    switch (i) {
#define SDM_SWZ(I) \
    case I: return (uint32_t)__builtin_amdgcn_ds_swizzle(v, kAnd | ((I) << 5));
        SDM_SWZ(0) SDM_SWZ(1) SDM_SWZ(2) SDM_SWZ(3) SDM_SWZ(4) SDM_SWZ(5) SDM_SWZ(6) SDM_SWZ(7)
        SDM_SWZ(8) SDM_SWZ(9) SDM_SWZ(10) SDM_SWZ(11) SDM_SWZ(12) SDM_SWZ(13) SDM_SWZ(14)
        SDM_SWZ(15) SDM_SWZ(16) SDM_SWZ(17) SDM_SWZ(18) SDM_SWZ(19) SDM_SWZ(20) SDM_SWZ(21)
        SDM_SWZ(22) SDM_SWZ(23) SDM_SWZ(24) SDM_SWZ(25) SDM_SWZ(26) SDM_SWZ(27) SDM_SWZ(28)
        SDM_SWZ(29) SDM_SWZ(30) SDM_SWZ(31)
#undef SDM_SWZ
    }
    return 0u;
}

// Value of x in lane `src` (any lane of the wave; src is a per-lane value).
__device__ __forceinline__ uint32_t lane_read(uint32_t x, int src)
{
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)x);
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
