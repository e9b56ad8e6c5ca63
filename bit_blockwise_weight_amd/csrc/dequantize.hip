// Dequantization kernel for gfx950.
//
// "LLM 相關知識" (technicalnotes, tag qlora), section 5 動態反量化: the 4-bit
// weight is restored to BF16 just before its matmul.  Definition used:
//     a'_j = absmax_j, or a'_j = RN_fp32(RN_fp32(q8_j * scale_{j/256}) + mean)
//     y_k  = RN_fp32(level[code_k] * a'_{k/B}),  written as fp32 or RNE-bf16.
// Two separate roundings (explicit _rn intrinsics, never fused).
//
// Work layout: lane l of a wave handles 8 consecutive elements (one 4-byte
// word of codes, one 16-byte bf16 store); 8 divides B, so the 8 elements share
// one block and one absmax.  The 16 levels sit in LDS, replicated 32 times and
// interleaved so the random code indexes of a wave never share a bank.
#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

constexpr int kThreads = 256;
constexpr int kCopies = 32;
constexpr int kUnroll = 2;
constexpr int kUnitElems = kWave * 8;

__device__ __forceinline__ float block_scale(const DeqArgs& a, int64_t blk) {
    if (!a.nested) return a.absmax[blk];
    const float sc = a.dq_scale[blk / QK_DQ_BLOCK];
    return __fadd_rn(__fmul_rn((float)a.q8[blk], sc), *a.dq_mean);
}

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DeqArgs a, void* __restrict__ out) {
    __shared__ float lev[16 * kCopies];
    // copy t % 32 of levels t / 32 and t / 32 + 8 (both loaded before either is written)
    static_assert(kCopies == 32 && kThreads == 256, "the fill assumes 32 copies and 256 threads");
    {
        const float l0 = a.levels[threadIdx.x / kCopies], l1 = a.levels[threadIdx.x / kCopies + 8];
        lev[threadIdx.x] = l0;
        lev[threadIdx.x + kThreads] = l1;
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int copy = lane & (kCopies - 1);
    const int64_t n = a.n;
    const int64_t nunits = (n + kUnitElems - 1) / kUnitElems;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);

    for (int64_t u0 = wave * kUnroll; u0 < nunits; u0 += nwaves * kUnroll) {
        uint32_t w[kUnroll];
        float sc[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t base = (u0 + k) * kUnitElems + lane * 8;
            w[k] = 0;
            sc[k] = 0.0f;
            if (base < n) {
                if (base + 8 <= n) {
                    w[k] = *reinterpret_cast<const uint32_t*>(a.codes + base / 2);
                } else {
                    const int64_t nbytes = (n + 1) / 2;
                    for (int j = 0; j < 4; ++j)
                        if (base / 2 + j < nbytes) w[k] |= (uint32_t)a.codes[base / 2 + j] << (8 * j);
                }
                sc[k] = block_scale(a, base >> a.blocksize_log2);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t base = (u0 + k) * kUnitElems + lane * 8;
            if (base >= n) continue;
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int shift = 8 * (i >> 1) + ((i & 1) ? 0 : 4);
                const uint32_t code = (w[k] >> shift) & 0xFu;
                y[i] = __fmul_rn(lev[code * kCopies + copy], sc[k]);
            }
            if (base + 8 <= n) {
                if constexpr (kBf16Out) {
                    uint4 o;
                    o.x = pack_bf16x2(y[0], y[1]);
                    o.y = pack_bf16x2(y[2], y[3]);
                    o.z = pack_bf16x2(y[4], y[5]);
                    o.w = pack_bf16x2(y[6], y[7]);
                    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + base) = o;
                } else {
                    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base);
                    p[0] = make_float4(y[0], y[1], y[2], y[3]);
                    p[1] = make_float4(y[4], y[5], y[6], y[7]);
                }
            } else {
                for (int i = 0; i < 8; ++i) {
                    if (base + i >= n) break;
                    if constexpr (kBf16Out) {
                        reinterpret_cast<uint16_t*>(out)[base + i] = (uint16_t)(pack_bf16x2(y[i], 0.0f) & 0xFFFFu);
                    } else {
                        reinterpret_cast<float*>(out)[base + i] = y[i];
                    }
                }
            }
        }
    }
}

}  // namespace



hipError_t launch_dequantize(const DeqArgs& a, void* out, int32_t out_dtype, hipStream_t s) {
    const int64_t nunits = (a.n + kUnitElems - 1) / kUnitElems;
    const int64_t waves_needed = (nunits + kUnroll - 1) / kUnroll;
    const int64_t wgs_needed = (waves_needed + (kThreads / kWave) - 1) / (kThreads / kWave);
    const int64_t cap = (int64_t)device_cu_count() * 16;
    const int grid = (int)(wgs_needed < cap ? wgs_needed : cap);
    if (out_dtype == QK_BF16)
        hipLaunchKernelGGL(dequantize_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a, out);
    else
        hipLaunchKernelGGL(dequantize_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a, out);
    return hipGetLastError();
}

}  // namespace qk
