// Blockwise 4-bit quantization kernel for gfx950.
//
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 QLoRA / NF4, 【例子】 and
// figure 2-2: per block of B elements take the absmax, divide the block by it,
// map each value to the nearest of the 16 levels, pack two codes per byte (first
// element in the high nibble).  Blocks run over the flattened tensor; the last
// one may be partial; a zero absmax gives t = +0.
//
// Work layout.  A wave handles "units" of 512 consecutive elements: lane l
// loads elements [8l, 8l+8) of the unit with one 16-byte load (bf16 / fp16) or
// two (fp32), so each load instruction reads 1 KB contiguous.  The B/8 lanes
// that share a block reduce its absmax with DPP moves (no LDS, no atomics).
// The grid is a few workgroups per CU (the LDS table is filled once per
// workgroup); each wave takes kUnroll consecutive units per iteration of a
// grid-stride loop and loads the next iteration's units before it processes the
// current ones, so two batches are in flight per lane.
//
// Division.  For bf16 and fp16 inputs t = RN(x/a) is computed from one IEEE
// reciprocal per block and Markstein's correction
//     q0 = x*r,  e = fma(-q0, a, x),  t = fma(e, r, q0),
// which equals the IEEE quotient bit for bit whenever 2^-36 <= a <= 2^64 and
// |x| >= a*2^-64 (checked exhaustively over every bf16 and every fp16 pair by
// the CPU test of the division).  Any lane holding an element outside that
// region redoes its 8 divisions with the IEEE sequence; fp32 inputs always use
// it.
//
// Nearest level.  t is binned by the low 24 bits of fmaf(t, S, S + 2^23); each
// bin of the LDS table holds at most one threshold T and the codes below and
// above it, so the code is one table read and one exact fp32 compare.  The table
// is replicated kLutCopies times, interleaved, and lane l reads copy l % 32, so
// the random bin indexes of a wave never collide in a bank.
#include "qk_internal.h"
#include "qk_device.h"
#include "qk_quant_io.h"

namespace qk {
namespace {

constexpr int kQThreads = 256;
constexpr int kLutCopies = 32;
constexpr int kUnroll = 1;
constexpr int kWgsPerCu = 8;
constexpr int kUnitElems = kWave * 8;

constexpr float kAMin = 0x1p-36f;
constexpr float kAMax = 0x1p64f;
constexpr float kXRel = 0x1p-64f;

template <typename InT, int B, bool kSorted>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const void* __restrict__ x, int64_t n,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ absmax,
                                                             QuantLut lut) {
    constexpr int G = B / 8;                       // lanes per block
    constexpr bool kFastDiv = !__is_same(InT, F32In);
    extern __shared__ uint2 lut_lds[];             // [nbins][kLutCopies]

    for (int i = threadIdx.x; i < lut.nbins * kLutCopies; i += kQThreads) {
        const int e = i / kLutCopies;
        lut_lds[i] = make_uint2(as_uint(lut.T[e]), lut.c[e]);
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t lane_off = (uint32_t)(lane & (kLutCopies - 1)) * 8u;
    constexpr uint32_t kBinStride = kLutCopies * 8u;
    const float S = lut.S, C = lut.C;
    const uint32_t bin_cap = 0x4B000000u + (uint32_t)(lut.nbins - 1);
    const int64_t nunits = (n + kUnitElems - 1) / kUnitElems;
    const int64_t nblocks = (n + B - 1) / B;
    const int64_t wave = (int64_t)blockIdx.x * (kQThreads / kWave) + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (kQThreads / kWave);
    const char* lds_bytes = reinterpret_cast<const char*>(lut_lds);

    // Raw input of kUnroll units per lane; the batch after the current one is loaded
    // before the current one is processed, so each wave keeps two batches in flight.
    using Raw = typename RawOf<InT>::type;
    Raw cur[kUnroll], nxt[kUnroll];
    auto load_batch = [&](int64_t u0, Raw (&r)[kUnroll]) {
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t unit = u0 + k < nunits ? u0 + k : nunits - 1;
            load_raw<InT>(x, n, unit * kUnitElems + lane * 8, r[k]);
        }
    };
    auto process = [&](int64_t u0, const Raw (&raw)[kUnroll]) {
        float v[kUnroll][8];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) unpack_raw<InT>(raw[k], v[k]);
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t unit = u0 + k;
            if (unit >= nunits) break;
            const int64_t base = unit * kUnitElems + lane * 8;
            float am = fmaxf(fmaxf(fmaxf(fabsf(v[k][0]), fabsf(v[k][1])), fmaxf(fabsf(v[k][2]), fabsf(v[k][3]))),
                             fmaxf(fmaxf(fabsf(v[k][4]), fabsf(v[k][5])), fmaxf(fabsf(v[k][6]), fabsf(v[k][7]))));
            am = group_max<G>(am);

            const float a_div = am == 0.0f ? 1.0f : am;   // zero block: x is +-0, t = +-0
            float t[8];
            bool ok = false;
            if constexpr (kFastDiv) {
                const bool fast_block = am >= kAMin && am <= kAMax;
                const float r = 1.0f / (fast_block ? am : 1.0f);
                const float x_lo = fast_block ? am * kXRel : __builtin_inff();
                ok = true;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float q0 = v[k][i] * r;
                    const float e = __builtin_fmaf(-q0, am, v[k][i]);
                    t[i] = __builtin_fmaf(e, r, q0);
                    ok = ok && (fabsf(v[k][i]) >= x_lo);
                }
            }
            if (!ok) {
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = v[k][i] / a_div;
            }

            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // |t| <= 1 gives the pattern 0x4B000000 + bin, bin in [0, 2S]; the min only
                // matters for non-finite input (outside the contract) and keeps the read in the table
                const uint32_t bin = min(as_uint(__builtin_fmaf(t[i], S, C)), bin_cap);
                const uint32_t addr = __umul24(bin, kBinStride) + lane_off;
                const uint2 ent = *reinterpret_cast<const uint2*>(lds_bytes + addr);
                uint32_t code;
                if constexpr (kSorted) {
                    code = ent.y + (t[i] >= as_float(ent.x) ? 1u : 0u);
                } else {
                    code = (ent.y >> (t[i] >= as_float(ent.x) ? 16u : 0u)) & 0xFu;
                }
                const int shift = 8 * (i >> 1) + ((i & 1) ? 0 : 4);
                word |= code << shift;
            }

            if ((unit + 1) * kUnitElems <= n) {
                *reinterpret_cast<uint32_t*>(codes + base / 2) = word;
            } else if (base < n) {
                // tail: codes of elements past n are 0, bytes past ceil(n/2) are not written
                const int64_t valid = n - base;          // 1..7 valid elements (or more)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t e0 = 2 * j;
                    if (e0 >= valid) break;
                    uint32_t byte = (word >> (8 * j)) & 0xFFu;
                    if (e0 + 1 >= valid) byte &= 0xF0u;
                    codes[base / 2 + j] = (uint8_t)byte;
                }
            }
            if ((lane % G) == 0 && base < n) {
                const int64_t blk = base / B;
                if (blk < nblocks) absmax[blk] = am;
            }
        }
    };
    // two batches in flight, the buffers alternating by name (a copy would wait for the load)
    const int64_t stride = nwaves * kUnroll;
    int64_t u0 = wave * kUnroll;
    if (u0 < nunits) load_batch(u0, cur);
    for (; u0 < nunits; u0 += 2 * stride) {
        if (u0 + stride < nunits) load_batch(u0 + stride, nxt);
        process(u0, cur);
        if (u0 + stride >= nunits) break;
        if (u0 + 2 * stride < nunits) load_batch(u0 + 2 * stride, cur);
        process(u0 + stride, nxt);
    }
}

int g_num_cus = 0;

int num_cus() {
    if (g_num_cus == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            g_num_cus = cus;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

template <typename InT, int B>
hipError_t launch_typed(const void* x, int64_t n, const QuantLut& lut, uint8_t* codes, float* absmax,
                        hipStream_t s) {
    const int64_t nunits = (n + kUnitElems - 1) / kUnitElems;
    const int64_t waves_needed = (nunits + kUnroll - 1) / kUnroll;
    const int64_t wgs_needed = (waves_needed + (kQThreads / kWave) - 1) / (kQThreads / kWave);
    const int64_t cap = (int64_t)num_cus() * kWgsPerCu;   // persistent: the LDS table is filled once per workgroup
    const int grid = (int)(wgs_needed < cap ? wgs_needed : cap);
    const size_t lds = (size_t)lut.nbins * kLutCopies * sizeof(uint2);
    if (lut.sorted)
        hipLaunchKernelGGL((quantize_kernel<InT, B, true>), dim3(grid), dim3(kQThreads), lds, s, x, n, codes,
                           absmax, lut);
    else
        hipLaunchKernelGGL((quantize_kernel<InT, B, false>), dim3(grid), dim3(kQThreads), lds, s, x, n, codes,
                           absmax, lut);
    return hipGetLastError();
}

template <typename InT>
hipError_t launch_bs(const void* x, int64_t n, int32_t blocksize, const QuantLut& lut, uint8_t* codes,
                     float* absmax, hipStream_t s) {
    switch (blocksize) {
        case 64: return launch_typed<InT, 64>(x, n, lut, codes, absmax, s);
        case 128: return launch_typed<InT, 128>(x, n, lut, codes, absmax, s);
        case 256: return launch_typed<InT, 256>(x, n, lut, codes, absmax, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int device_cu_count() { return num_cus(); }

hipError_t launch_quantize(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize, const QuantLut& lut,
                           uint8_t* codes, float* absmax, hipStream_t s) {
    switch (x_dtype) {
        case QK_BF16: return launch_bs<Bf16In>(x, n, blocksize, lut, codes, absmax, s);
        case QK_F16: return launch_bs<F16In>(x, n, blocksize, lut, codes, absmax, s);
        case QK_F32: return launch_bs<F32In>(x, n, blocksize, lut, codes, absmax, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qk
