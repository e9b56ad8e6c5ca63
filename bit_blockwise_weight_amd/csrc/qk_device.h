// Device helpers shared by the gfx950 kernels of libqk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

constexpr int kWave = 64;

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 pair in a dword -> two fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Cross-lane max within aligned groups of `G` lanes (G = 1..32), every lane of
// the group receives the result.  DPP for the steps inside a row of 16 lanes,
// a swizzle for the step across two rows.
template <int G>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (G >= 2) {   // xor 1: quad_perm [1,0,3,2]
        v = fmaxf(v, as_float(__builtin_amdgcn_mov_dpp(as_uint(v), 0xB1, 0xF, 0xF, false)));
    }
    if constexpr (G >= 4) {   // xor 2: quad_perm [2,3,0,1]
        v = fmaxf(v, as_float(__builtin_amdgcn_mov_dpp(as_uint(v), 0x4E, 0xF, 0xF, false)));
    }
    if constexpr (G >= 8) {   // row_half_mirror: lane i <- 7-i within 8 lanes
        v = fmaxf(v, as_float(__builtin_amdgcn_mov_dpp(as_uint(v), 0x141, 0xF, 0xF, false)));
    }
    if constexpr (G >= 16) {  // row_mirror: lane i <- 15-i within 16 lanes
        v = fmaxf(v, as_float(__builtin_amdgcn_mov_dpp(as_uint(v), 0x140, 0xF, 0xF, false)));
    }
    if constexpr (G >= 32) {  // swizzle, bit-mask mode: lane i <- i ^ 16 within 32 lanes
        v = fmaxf(v, as_float(__builtin_amdgcn_ds_swizzle(as_uint(v), 0x401F)));
    }
    return v;
}

// The same for unsigned integers (for instance the bit patterns of non-negative
// floats, whose order is the order of the values): no NaN canonicalization, and
// each move folds into its max instruction (v_max_u32 with a DPP source).  The
// folding needs the move's old value to be the identity of the max (0); every lane
// has a source in these patterns, so the old value is never used.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if constexpr (G >= 2) v = max((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true), v);
    if constexpr (G >= 4) v = max((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true), v);
    if constexpr (G >= 8) v = max((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true), v);
    if constexpr (G >= 16) v = max((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true), v);
    if constexpr (G >= 32) v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
    return v;
}

}  // namespace qk
