// 8-bit blockwise quantization and dequantization with a 256-level map, gfx950.
//
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.3 8-bit Optimizers, 【原理】 and
// figure 2-3: optimizer states are cut into blocks (2048 elements in the figure),
// each block is scaled by its own absmax and every value is mapped to one of 256
// non-uniform levels (the dynamic map), one code per byte.  The decision is the
// exact nearest level with ties to the smaller code, as in the 4-bit kernel.
//
// Quantize.  A wave takes a "unit" of max(B, 512) consecutive elements, 8 per
// lane per 512 (16-bit inputs: 8 consecutive elements, one 16-byte load; fp32:
// two runs of 4, 256 apart, two 16-byte loads), so each load instruction reads
// 1 KB contiguous.  The block absmax is reduced with DPP / swizzle inside the
// lanes of a block, or over the whole wave (two readlanes).  t = RN(x / a): bf16 / fp16 inputs take the reciprocal +
// Markstein correction where it is exact (the region the CPU division test
// covers), fp32 inputs the IEEE division.  The code comes from a per-workgroup
// LDS bin table built at kernel start from the host's validated thresholds: one
// fma for the bin, one 8-byte table read, one compare.  Persistent grid, each
// wave loads the next unit before it processes the current one.
//
// Dequantize.  y = RN(l[code] * a): the level table sits in LDS in 32
// interleaved copies (lane l reads copy l % 32: no bank conflicts); each load and
// store instruction of a wave covers contiguous memory (see the kernel).
#include "qk_internal.h"
#include "qk_device.h"
#include "qk_quant_io.h"

namespace qk {
namespace {

constexpr int kThreads = 256;
constexpr int kWgsPerCu8 = 4;
constexpr float kAMin8 = 0x1p-36f;
constexpr float kAMax8 = 0x1p64f;
constexpr float kXRel8 = 0x1p-64f;

// least binary32 t with bin(t) >= b, bin(t) = round-half-even(t S + S), S a power of two
__device__ __forceinline__ float bin_start(int b, float S) {
    const float v = ((float)b - S - 0.5f) / S;     // exact: a half-integer over a power of two, never 0
    const uint32_t u = as_uint(v);
    return (b & 1) ? as_float(v > 0.0f ? u + 1u : u - 1u) : v;   // odd b: the next binary32 value up
}

template <typename InT, int B>
__global__ __launch_bounds__(kThreads) void quantize8_kernel(const void* __restrict__ x, int64_t n,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ absmax, QuantLut8 lut) {
    constexpr int E = B < 512 ? 512 : B;           // elements per unit
    constexpr int U = E / 512;                     // 8-element groups per lane per unit
    constexpr int G = B < 512 ? B / 8 : 64;        // lanes per block
    constexpr bool kFastDiv = !__is_same(InT, F32In);
    __shared__ float thr[256];
    __shared__ uint8_t cof[256];
    __shared__ uint2 tab[kLut8MaxBins];

    const int tid = threadIdx.x;
    thr[tid] = tid < lut.nthr ? lut.T[tid < 255 ? tid : 254] : 2.0f;
    cof[tid] = lut.code_of[tid];
    __syncthreads();
    const float S = lut.S, C = lut.C;
    for (int b = tid; b < lut.nbins; b += kThreads) {
        const float tb = bin_start(b, S), tn = bin_start(b + 1, S);
        int lo = 0;                                 // thresholds <= tb (increasing order)
        for (int step = 128; step > 0; step >>= 1)
            if (lo + step <= lut.nthr && thr[lo + step - 1] <= tb) lo += step;
        const bool inside = lo < lut.nthr && thr[lo] < tn;
        const uint32_t clo = cof[lo], chi = inside ? cof[lo + 1] : clo;
        tab[b] = make_uint2(as_uint(inside ? thr[lo] : 2.0f), clo | (chi << 16));
    }
    __syncthreads();

    const int lane = tid & (kWave - 1);
    const uint32_t bin_cap = 0x4B000000u + (uint32_t)(lut.nbins - 1);
    const int64_t nunits = (n + E - 1) / E;
    const int64_t nblocks = (n + B - 1) / B;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);

    // fp32: lane l holds elements [512 u + 4 l, + 4) and [512 u + 256 + 4 l, + 4) (two
    // 16-byte loads, each contiguous over the wave); 16-bit types: [512 u + 8 l, + 8)
    constexpr bool kSplit = __is_same(InT, F32In);
    auto pos = [&](int64_t unit, int u, int i) -> int64_t {
        if constexpr (kSplit) return unit * E + 512 * u + (i < 4 ? 4 * lane + i : 256 + 4 * lane + (i - 4));
        else return unit * E + 512 * u + 8 * lane + i;
    };
    using Raw = typename RawOf<InT>::type;
    Raw cur[U], nxt[U];
    auto load_unit = [&](int64_t unit, Raw (&r)[U]) {
        unit = unit < nunits ? unit : nunits - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (kSplit) {
                const float* xf = reinterpret_cast<const float*>(x);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int64_t e0 = pos(unit, u, 4 * hh);
                    if (e0 + 4 <= n) {
                        r[u][hh] = *reinterpret_cast<const uint4*>(xf + e0);
                    } else {
                        uint32_t w4[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) w4[k] = e0 + k < n ? as_uint(xf[e0 + k]) : 0u;
                        r[u][hh] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                    }
                }
            } else {
                load_raw<InT>(x, n, pos(unit, u, 0), r[u]);
            }
        }
    };
    auto wave_max = [&](float v) {
        v = group_max<32>(v);
        return fmaxf(as_float(__builtin_amdgcn_readlane(as_uint(v), 0)), as_float(__builtin_amdgcn_readlane(as_uint(v), 32)));
    };
    // with fp32 input and B = 256 the two halves of a lane's 8 elements are two blocks
    constexpr bool kTwoBlocks = kSplit && B == 256;
    auto process = [&](int64_t unit, const Raw (&raw)[U]) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) unpack_raw<InT>(raw[u], v[u]);
        float amh[2] = {0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) amh[kTwoBlocks && i >= 4] = fmaxf(amh[kTwoBlocks && i >= 4], fabsf(v[u][i]));
        if constexpr (kTwoBlocks) {
            amh[0] = wave_max(amh[0]);
            amh[1] = wave_max(amh[1]);
        } else if constexpr (G == 64 || kSplit) {
            amh[0] = amh[1] = wave_max(amh[0]);
        } else {
            amh[0] = amh[1] = group_max<G>(amh[0]);
        }
        float adiv[2], r[2] = {1.0f, 1.0f}, x_lo[2] = {__builtin_inff(), __builtin_inff()};
        bool fast[2] = {false, false};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            adiv[hh] = amh[hh] == 0.0f ? 1.0f : amh[hh];   // zero block: x is +-0, t = +-0
            if constexpr (kFastDiv) {
                fast[hh] = amh[hh] >= kAMin8 && amh[hh] <= kAMax8;
                r[hh] = 1.0f / (fast[hh] ? amh[hh] : 1.0f);
                x_lo[hh] = fast[hh] ? amh[hh] * kXRel8 : __builtin_inff();
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float t[8];
            bool ok = fast[0];
            if constexpr (kFastDiv) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float q0 = v[u][i] * r[0];
                    const float e = __builtin_fmaf(-q0, amh[0], v[u][i]);
                    t[i] = __builtin_fmaf(e, r[0], q0);
                    ok = ok && (fabsf(v[u][i]) >= x_lo[0]);
                }
            }
            if (!ok) {
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = v[u][i] / adiv[kTwoBlocks && i >= 4];
            }
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // |t| <= 1 gives 0x4B000000 + bin, bin in [0, 2S]; the min keeps non-finite input in the table
                const uint32_t bin = min(as_uint(__builtin_fmaf(t[i], S, C)), bin_cap) - 0x4B000000u;
                const uint2 ent = tab[bin];
                const uint32_t code = (ent.y >> (t[i] >= as_float(ent.x) ? 16u : 0u)) & 0xFFu;
                w[i >> 2] |= code << (8 * (i & 3));
            }
            if constexpr (kSplit) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int64_t e0 = pos(unit, u, 4 * hh);
                    if (e0 + 4 <= n) *reinterpret_cast<uint32_t*>(codes + e0) = w[hh];
                    else for (int k = 0; k < 4 && e0 + k < n; ++k) codes[e0 + k] = (uint8_t)(w[hh] >> (8 * k));
                }
            } else {
                const int64_t base = pos(unit, u, 0);
                if (base + 8 <= n) {
                    *reinterpret_cast<uint2*>(codes + base) = make_uint2(w[0], w[1]);
                } else if (base < n) {
                    for (int i = 0; i < 8 && base + i < n; ++i) codes[base + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
                }
                if constexpr (G < 64) {
                    if ((lane % G) == 0 && base < n) absmax[base / B] = amh[0];
                }
            }
        }
        if constexpr (kTwoBlocks) {
            if (lane == 0) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    if (2 * unit + hh < nblocks) absmax[2 * unit + hh] = amh[hh];
            }
        } else if constexpr (G == 64) {
            if (lane == 0 && unit < nblocks) absmax[unit] = amh[0];
        }
    };
    // the next unit is loaded before the current one is processed; buffers alternate by name
    int64_t unit = wave;
    if (unit < nunits) load_unit(unit, cur);
    for (; unit < nunits; unit += 2 * nwaves) {
        if (unit + nwaves < nunits) load_unit(unit + nwaves, nxt);
        process(unit, cur);
        if (unit + nwaves >= nunits) break;
        if (unit + 2 * nwaves < nunits) load_unit(unit + 2 * nwaves, cur);
        process(unit + nwaves, nxt);
    }
}

struct Levels256 {
    float v[256];
};

// A wave takes 1024 consecutive elements per iteration in Q steps of 64 V elements:
// in step q lane l owns elements [64 V q + V l, + V), so every code load and every
// result store of the wave is contiguous (fp32: V = 4, 16-byte stores; bf16: V = 8).
template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void dequantize8_kernel(const uint8_t* __restrict__ codes,
                                                               const float* __restrict__ absmax, int64_t n,
                                                               int32_t blocksize_log2, Levels256 lv,
                                                               void* __restrict__ out) {
    constexpr int kCopies = 32;
    constexpr int V = kBf16Out ? 8 : 4;
    constexpr int Q = 1024 / (64 * V);
    __shared__ float tab[256 * kCopies];
    {
        // copy t % 32 of the levels t / 32 + 8 j, j < 32: all 32 loads are issued before the
        // first write, so the fill costs one memory round trip
        static_assert(kCopies == 32 && kThreads == 256, "the fill assumes 32 copies and 256 threads");
        const int c = threadIdx.x & (kCopies - 1), v0 = threadIdx.x / kCopies;
        float lvv[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) lvv[j] = lv.v[v0 + 8 * j];
#pragma unroll
        for (int j = 0; j < 32; ++j) tab[(v0 + 8 * j) * kCopies + c] = lvv[j];
    }
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int copy = lane & (kCopies - 1);
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
    const int64_t ngroups = (n + 1023) / 1024;
    for (int64_t g = wave; g < ngroups; g += nwaves) {
        uint32_t w[Q][V / 4];
        float a[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t base = g * 1024 + 64 * V * q + V * lane;
            if (base + V <= n) {
                if constexpr (V == 8) {
                    const uint2 c = *reinterpret_cast<const uint2*>(codes + base);
                    w[q][0] = c.x;
                    w[q][1] = c.y;
                } else {
                    w[q][0] = *reinterpret_cast<const uint32_t*>(codes + base);
                }
            } else {
#pragma unroll
                for (int k = 0; k < V / 4; ++k) w[q][k] = 0u;
                for (int i = 0; i < V && base + i < n; ++i) w[q][i >> 2] |= (uint32_t)codes[base + i] << (8 * (i & 3));
            }
            a[q] = absmax[(base < n ? base : n - 1) >> blocksize_log2];   // V elements of one block (B >= 256)
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t base = g * 1024 + 64 * V * q + V * lane;
            if (base >= n) continue;
            float y[V];
#pragma unroll
            for (int i = 0; i < V; ++i)
                y[i] = __fmul_rn(tab[((w[q][i >> 2] >> (8 * (i & 3))) & 0xFFu) * kCopies + copy], a[q]);
            if (base + V <= n) {
                if constexpr (kBf16Out) {
                    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + base) =
                        make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                   pack_bf16x2(y[6], y[7]));
                } else {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base) = make_float4(y[0], y[1], y[2], y[3]);
                }
            } else {
                for (int i = 0; i < V && base + i < n; ++i) {
                    if constexpr (kBf16Out)
                        reinterpret_cast<uint16_t*>(out)[base + i] = (uint16_t)(pack_bf16x2(y[i], 0.0f) & 0xFFFFu);
                    else
                        reinterpret_cast<float*>(out)[base + i] = y[i];
                }
            }
        }
    }
}

template <typename InT, int B>
hipError_t launch_q8(const void* x, int64_t n, const QuantLut8& lut, uint8_t* codes, float* absmax, hipStream_t s) {
    constexpr int E = B < 512 ? 512 : B;
    const int64_t nunits = (n + E - 1) / E;
    const int64_t wgs_needed = (nunits + (kThreads / kWave) - 1) / (kThreads / kWave);
    const int64_t cap = (int64_t)device_cu_count() * kWgsPerCu8;
    const int grid = (int)(wgs_needed < cap ? wgs_needed : cap);
    hipLaunchKernelGGL((quantize8_kernel<InT, B>), dim3(grid), dim3(kThreads), 0, s, x, n, codes, absmax, lut);
    return hipGetLastError();
}

template <typename InT>
hipError_t launch_q8_bs(const void* x, int64_t n, int32_t blocksize, const QuantLut8& lut, uint8_t* codes,
                        float* absmax, hipStream_t s) {
    switch (blocksize) {
        case 256: return launch_q8<InT, 256>(x, n, lut, codes, absmax, s);
        case 512: return launch_q8<InT, 512>(x, n, lut, codes, absmax, s);
        case 1024: return launch_q8<InT, 1024>(x, n, lut, codes, absmax, s);
        case 2048: return launch_q8<InT, 2048>(x, n, lut, codes, absmax, s);
        case 4096: return launch_q8<InT, 4096>(x, n, lut, codes, absmax, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize8(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize, const QuantLut8& lut,
                            uint8_t* codes, float* absmax, hipStream_t s) {
    switch (x_dtype) {
        case QK_BF16: return launch_q8_bs<Bf16In>(x, n, blocksize, lut, codes, absmax, s);
        case QK_F16: return launch_q8_bs<F16In>(x, n, blocksize, lut, codes, absmax, s);
        case QK_F32: return launch_q8_bs<F32In>(x, n, blocksize, lut, codes, absmax, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequantize8(const uint8_t* codes, const float* absmax, int64_t n, int32_t blocksize,
                              const float levels[256], void* out, int32_t out_dtype, hipStream_t s) {
    Levels256 lv;
    for (int i = 0; i < 256; ++i) lv.v[i] = levels[i];
    int lg = 0;
    while ((1 << lg) < blocksize) ++lg;
    const int64_t ngroups = (n + 1023) / 1024;
    const int64_t wgs_needed = (ngroups + (kThreads / kWave) - 1) / (kThreads / kWave);
    const int64_t cap = (int64_t)device_cu_count() * kWgsPerCu8;
    const int grid = (int)(wgs_needed < cap ? wgs_needed : cap);
    if (out_dtype == QK_BF16)
        hipLaunchKernelGGL((dequantize8_kernel<true>), dim3(grid), dim3(kThreads), 0, s, codes, absmax, n, lg, lv, out);
    else if (out_dtype == QK_F32)
        hipLaunchKernelGGL((dequantize8_kernel<false>), dim3(grid), dim3(kThreads), 0, s, codes, absmax, n, lg, lv, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace qk
