// Input loading shared by the blockwise quantize kernels of libqk (gfx950).
//
// A lane reads 8 consecutive elements at a time: one 16-byte load for bf16 /
// fp16, two for fp32; a lane whose 8 elements run past n loads them one by one
// (zeros past n).
#pragma once

#include "qk_device.h"

namespace qk {
namespace {

struct Bf16In {};
struct F16In {};
struct F32In {};

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Raw 8-element input of one lane: one 16-byte word for 16-bit types, two for fp32.
// A lane whose 8 elements run past n loads them one by one (zeros past n).
template <typename T> struct RawOf { typedef uint4 type; };
template <> struct RawOf<F32In> { typedef uint4 type[2]; };

template <typename T>
__device__ __forceinline__ void load_raw(const void* x, int64_t n, int64_t base, typename RawOf<T>::type& r) {
    if constexpr (__is_same(T, F32In)) {
        if (base + 8 <= n) {
            const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + base);
            r[0] = p[0];
            r[1] = p[1];
        } else {
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = (base + i < n) ? as_uint(reinterpret_cast<const float*>(x)[base + i]) : 0u;
            r[0] = make_uint4(w[0], w[1], w[2], w[3]);
            r[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    } else {
        if (base + 8 <= n) {
            r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + base);
        } else {
            uint32_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = (base + i < n) ? (uint32_t)reinterpret_cast<const uint16_t*>(x)[base + i] : 0u;
            r = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        }
    }
}

// The same for a lane whose 8 elements are known to be in range: no branch, so the
// compiler can leave the load in flight across unrelated code.
// The loads are nontemporal: the input is streamed once.
typedef unsigned int u32x4_stream_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 stream_load16(const void* p) {
    const u32x4_stream_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_stream_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
__device__ __forceinline__ void load_raw_full(const void* x, int64_t base, typename RawOf<T>::type& r) {
    if constexpr (__is_same(T, F32In)) {
        const float* p = reinterpret_cast<const float*>(x) + base;
        r[0] = stream_load16(p);
        r[1] = stream_load16(p + 4);
    } else {
        r = stream_load16(reinterpret_cast<const uint16_t*>(x) + base);
    }
}

template <typename T>
__device__ __forceinline__ void unpack_raw(const typename RawOf<T>::type& r, float v[8]) {
    if constexpr (__is_same(T, F32In)) {
        v[0] = as_float(r[0].x); v[1] = as_float(r[0].y); v[2] = as_float(r[0].z); v[3] = as_float(r[0].w);
        v[4] = as_float(r[1].x); v[5] = as_float(r[1].y); v[6] = as_float(r[1].z); v[7] = as_float(r[1].w);
    } else if constexpr (__is_same(T, F16In)) {
        v[0] = h2f(r.x & 0xFFFF); v[1] = h2f(r.x >> 16);
        v[2] = h2f(r.y & 0xFFFF); v[3] = h2f(r.y >> 16);
        v[4] = h2f(r.z & 0xFFFF); v[5] = h2f(r.z >> 16);
        v[6] = h2f(r.w & 0xFFFF); v[7] = h2f(r.w >> 16);
    } else {
        v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
        v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
        v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
        v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
    }
}

// Largest and smallest |x| of a lane's 8 elements, from the raw words: the bit
// pattern of a non-negative float orders like the value, so both are integer
// max / min of the patterns with the sign cleared (two 16-bit halves at a time for
// bf16 / fp16).  Finite input.
template <typename T>
__device__ __forceinline__ void abs_range_raw(const typename RawOf<T>::type& r, float& amax, float& amin) {
    if constexpr (__is_same(T, F32In)) {
        const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
        uint32_t hi = w[0] & 0x7FFFFFFFu, lo = hi;
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            const uint32_t a = w[i] & 0x7FFFFFFFu;
            hi = max(hi, a);
            lo = min(lo, a);
        }
        amax = as_float(hi);
        amin = as_float(lo);
    } else {
        typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
        const u16x2_t a0 = __builtin_bit_cast(u16x2_t, r.x & 0x7FFF7FFFu);
        const u16x2_t a1 = __builtin_bit_cast(u16x2_t, r.y & 0x7FFF7FFFu);
        const u16x2_t a2 = __builtin_bit_cast(u16x2_t, r.z & 0x7FFF7FFFu);
        const u16x2_t a3 = __builtin_bit_cast(u16x2_t, r.w & 0x7FFF7FFFu);
        const u16x2_t mx = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1), __builtin_elementwise_max(a2, a3));
        const u16x2_t mn = __builtin_elementwise_min(__builtin_elementwise_min(a0, a1), __builtin_elementwise_min(a2, a3));
        const uint32_t hi = max((uint32_t)mx.x, (uint32_t)mx.y);
        const uint32_t lo = min((uint32_t)mn.x, (uint32_t)mn.y);
        if constexpr (__is_same(T, F16In)) {
            amax = h2f(hi);
            amin = h2f(lo);
        } else {
            amax = as_float(hi << 16);
            amin = as_float(lo << 16);
        }
    }
}

}  // namespace
}  // namespace qk
