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
// one block and one absmax.  A wave takes two 512-element units per turn; a turn
// whose elements all exist loads and stores without conditions (the code loads
// nontemporal), the last turns go element by element.  The 16 levels sit in LDS,
// replicated 32 times and interleaved so the random code indexes of a wave never
// share a bank.
#include <cstring>
#include <vector>

#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

constexpr int kThreads = 256;
constexpr int kCopies = 32;
constexpr int kUnroll = 2;
constexpr int kUnitElems = kWave * 8;
constexpr int kMaxDeqGroup = 16;

__device__ __forceinline__ float block_scale(const DeqArgs& a, int64_t blk) {
    if (!a.nested) return a.absmax[blk];
    const float sc = a.dq_scale[blk / QK_DQ_BLOCK];
    return __fadd_rn(__fmul_rn((float)a.q8[blk], sc), *a.dq_mean);
}

// The arrays of one launch (a single call is a group of one); all of them have the
// same level table.  Array t owns the global turns [turn0[t], turn0[t + 1]).
struct DeqGroup {
    DeqArgs a[kMaxDeqGroup];
    void* out[kMaxDeqGroup];
    int64_t turn0[kMaxDeqGroup + 1];
    int32_t count;
};

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DeqGroup g) {
    __shared__ float lev[16 * kCopies];
    // copy t % 32 of levels t / 32 and t / 32 + 8 (both loaded before either is written)
    static_assert(kCopies == 32 && kThreads == 256, "the fill assumes 32 copies and 256 threads");
    {
        const float l0 = g.a[0].levels[threadIdx.x / kCopies], l1 = g.a[0].levels[threadIdx.x / kCopies + 8];
        lev[threadIdx.x] = l0;
        lev[threadIdx.x + kThreads] = l1;
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int copy = lane & (kCopies - 1);
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);

    // the 8 values of a code word, and their 16-byte (bf16) or 2 x 16-byte (fp32) store
    auto emit8 = [&](uint32_t cw, float scale, float (&y)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int shift = 8 * (i >> 1) + ((i & 1) ? 0 : 4);
            const uint32_t code = (cw >> shift) & 0xFu;
            y[i] = __fmul_rn(lev[code * kCopies + copy], scale);
        }
    };
    auto store8 = [&](void* out, int64_t base, const float (&y)[8]) {
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
    };

    // a wave takes its turns in increasing order, so the array cursor only moves
    // forward and the array's descriptor is read only when it crosses into the next
    const int64_t nturns = g.turn0[g.count];
    int k = 0;
    int64_t k_end = g.turn0[1];
    DeqArgs a = g.a[0];
    void* out = g.out[0];
    for (int64_t t = wave; t < nturns; t += nwaves) {
        if (t >= k_end) {
            while (t >= g.turn0[k + 1]) ++k;
            k_end = g.turn0[k + 1];
            a = g.a[k];
            out = g.out[k];
        }
        const int64_t n = a.n;
        const int64_t u0 = (t - g.turn0[k]) * kUnroll;
        uint32_t w[kUnroll];
        float sc[kUnroll];
        if ((u0 + kUnroll) * kUnitElems <= n) {
            // every element of the turn exists: unconditional loads (nontemporal: each
            // code is read once) and stores.  Measured on a 70B-shaped layer, 623 -> 497 us
            // against the guarded form below (4.9 TB/s, at the ceiling of a stream that
            // reads 4 bytes per 16 written).
#pragma unroll
            for (int kk = 0; kk < kUnroll; ++kk) {
                const int64_t base = (u0 + kk) * kUnitElems + lane * 8;
                w[kk] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.codes + base / 2));
                sc[kk] = block_scale(a, base >> a.blocksize_log2);
            }
#pragma unroll
            for (int kk = 0; kk < kUnroll; ++kk) {
                const int64_t base = (u0 + kk) * kUnitElems + lane * 8;
                float y[8];
                emit8(w[kk], sc[kk], y);
                store8(out, base, y);
            }
            continue;
        }
#pragma unroll
        for (int kk = 0; kk < kUnroll; ++kk) {
            const int64_t base = (u0 + kk) * kUnitElems + lane * 8;
            w[kk] = 0;
            sc[kk] = 0.0f;
            if (base < n) {
                if (base + 8 <= n) {
                    w[kk] = *reinterpret_cast<const uint32_t*>(a.codes + base / 2);
                } else {
                    const int64_t nbytes = (n + 1) / 2;
                    for (int j = 0; j < 4; ++j)
                        if (base / 2 + j < nbytes) w[kk] |= (uint32_t)a.codes[base / 2 + j] << (8 * j);
                }
                sc[kk] = block_scale(a, base >> a.blocksize_log2);
            }
        }
#pragma unroll
        for (int kk = 0; kk < kUnroll; ++kk) {
            const int64_t base = (u0 + kk) * kUnitElems + lane * 8;
            if (base >= n) continue;
            float y[8];
            emit8(w[kk], sc[kk], y);
            if (base + 8 <= n) {
                store8(out, base, y);
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

hipError_t launch_group(const DeqGroup& g, int32_t out_dtype, hipStream_t s) {
    const int64_t wgs_needed = (g.turn0[g.count] + (kThreads / kWave) - 1) / (kThreads / kWave);
    const int64_t cap = (int64_t)device_cu_count() * 16;
    const int grid = (int)(wgs_needed < cap ? wgs_needed : cap);
    if (out_dtype == QK_BF16)
        hipLaunchKernelGGL(dequantize_kernel<true>, dim3(grid), dim3(kThreads), 0, s, g);
    else
        hipLaunchKernelGGL(dequantize_kernel<false>, dim3(grid), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

int64_t turns_of(int64_t n) { return ((n + kUnitElems - 1) / kUnitElems + kUnroll - 1) / kUnroll; }

}  // namespace

hipError_t launch_dequantize(const DeqArgs& a, void* out, int32_t out_dtype, hipStream_t s) {
    DeqItem it{a, out};
    return launch_dequantize_group(&it, 1, out_dtype, s);
}

hipError_t launch_dequantize_group(const DeqItem* items, int32_t count, int32_t out_dtype, hipStream_t s) {
    // arrays that share a level table go together, up to kMaxDeqGroup per launch
    std::vector<bool> used(count, false);
    for (int32_t f = 0; f < count; ++f) {
        if (used[f]) continue;
        DeqGroup g;
        std::memset(&g, 0, sizeof(g));
        int64_t turns = 0;
        for (int32_t i = f; i < count && g.count < kMaxDeqGroup; ++i) {
            if (used[i] || std::memcmp(items[i].a.levels, items[f].a.levels, sizeof(items[f].a.levels)) != 0) continue;
            g.a[g.count] = items[i].a;
            g.out[g.count] = items[i].out;
            g.turn0[g.count] = turns;
            turns += turns_of(items[i].a.n);
            ++g.count;
            used[i] = true;
        }
        g.turn0[g.count] = turns;
        const hipError_t e = launch_group(g, out_dtype, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}


}  // namespace qk
