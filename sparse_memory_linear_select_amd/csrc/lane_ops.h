// Lane exchanges of a 64-lane wavefront that avoid the LDS crossbar
// (ds_bpermute): DPP moves and the gfx950 permlane swaps, a few cycles each
// where a crossbar round trip takes about a hundred.
#pragma once

#include "sdm_internal.h"

namespace sdm {
namespace {

// x of lane l ^ m.  m is a compile-time constant at every call (the
// callers' loops are unrolled): the DPP controls must be immediates.
//   m = 1, 2   one DPP quad permutation;
//   m = 4      row_shl:4 into banks 0 and 2 (lanes with bit 2 clear), then
//              row_shr:4 into banks 1 and 3 (bank = 4 lanes of a 16-lane row);
//   m = 8      row_ror:8 (a rotation by half of the 16-lane row);
//   m = 16, 32 see pair_vals.
// Every lane is written (m = 4: the second move writes the banks the first
// leaves out), so the moves take no old value and need no copy of one.
__device__ __forceinline__ uint32_t dpp_xor(uint32_t x, int m)
{
    switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
    case 4: {
        const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x104, 0xF, 0x5, false);
        return __builtin_amdgcn_update_dpp(y, x, 0x114, 0xF, 0xA, false);
    }
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);
    }
}

// m = 16 or 32: the gfx950 permlane swaps give every lane both values of its
// pair {l, l ^ m}: lo the lower lane's, hi the upper lane's.
__device__ __forceinline__ void pair_vals(uint32_t x, int m, uint32_t &lo, uint32_t &hi)
{
    if (m == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        lo = r[0];
        hi = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        lo = r[0];
        hi = r[1];
    }
}

// x + x of lane ^ m (a butterfly step of a sum), without the LDS crossbar.
// Both lanes of a pair add the same two values (in either order: the same
// float).
__device__ __forceinline__ float xor_add(float x, int m)
{
    if (m >= 16) {
        uint32_t lo, hi;
        pair_vals(__float_as_uint(x), m, lo, hi);
        return __uint_as_float(lo) + __uint_as_float(hi);
    }
    return x + __uint_as_float(dpp_xor(__float_as_uint(x), m));
}

}  // namespace
}  // namespace sdm
