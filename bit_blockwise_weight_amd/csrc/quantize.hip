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
// workgroup); each wave walks the full units with a grid stride and loads its
// next unit before it processes the current one, so two units are in flight per
// lane.  Those loads are unconditional (no branch between a load and its use, so
// the compiler's wait leaves the next unit's load outstanding); the partial last
// unit, if any, is done after the loop by one wave with per-element loads.
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
#include <type_traits>

#include "qk_internal.h"
#include "qk_device.h"
#include "qk_quant_io.h"

namespace qk {
namespace {

constexpr int kQThreads = 256;
constexpr int kLutCopies = 32;
constexpr int kWgsPerCu = 8;
constexpr int kUnitElems = kWave * 8;
constexpr int kBatch = 2;                 // consecutive units a wave loads per turn

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

    {
        // copy t % 32 of the entries t / 32 + 8 j: every load is issued before the first
        // write (indexes past the last bin re-read it), so the fill costs one memory round
        // trip, not one per entry
        static_assert(kLutCopies == 32 && kQThreads == 256, "the fill assumes 32 copies and 256 threads");
        constexpr int kFill = (kLutMaxBins + 7) / 8;
        const int c = threadIdx.x & (kLutCopies - 1), e0 = threadIdx.x / kLutCopies;
        uint2 ent[kFill];
#pragma unroll
        for (int j = 0; j < kFill; ++j) {
            const int e = min(e0 + 8 * j, lut.nbins - 1);
            ent[j] = make_uint2(as_uint(lut.T[e]), lut.c[e]);
        }
#pragma unroll
        for (int j = 0; j < kFill; ++j) {
            if (e0 + 8 * j < lut.nbins) lut_lds[(e0 + 8 * j) * kLutCopies + c] = ent[j];
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t lane_off = (uint32_t)(lane & (kLutCopies - 1)) * 8u;
    constexpr uint32_t kBinStride = kLutCopies * 8u;
    const float S = lut.S, C = lut.C;
    const uint32_t bin_cap = 0x4B000000u + (uint32_t)(lut.nbins - 1);
    const int64_t nfull = n / kUnitElems;          // units whose 512 elements are all in range
    // uniform in the wave: the loop below is then scalar control flow
    const int64_t wave = (int64_t)blockIdx.x * (kQThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kQThreads / kWave);
    const char* lds_bytes = reinterpret_cast<const char*>(lut_lds);

    const int64_t nbatches = nfull / kBatch;        // batches of kBatch full units
    const int64_t nunits = (n + kUnitElems - 1) / kUnitElems;

    using Raw = typename RawOf<InT>::type;
    // A batch: one unconditional load per lane and unit (the batch index is clamped, so
    // the prefetch past the last batch re-reads it); no branch separates a load from
    // the code that waits for it, so the other batch's loads stay in flight meanwhile.
    auto load_batch = [&](int64_t bi, Raw (&r)[kBatch]) {
        const int64_t bc = bi < nbatches ? bi : nbatches - 1;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) load_raw_full<InT>(x, (bc * kBatch + k) * kUnitElems + lane * 8, r[k]);
    };
    auto process = [&](int64_t unit, const Raw& raw, auto tail_tag) {
        constexpr bool kTail = decltype(tail_tag)::value;
        float v[8];
        unpack_raw<InT>(raw, v);
        const int64_t base = unit * kUnitElems + lane * 8;
        float am, mn;
        abs_range_raw<InT>(raw, am, mn);
        am = as_float(group_max_u32<G>(as_uint(am)));

        float t[8];
        bool ok = false;
        if constexpr (kFastDiv) {
            const bool fast_block = am >= kAMin && am <= kAMax;
            const float r = 1.0f / (fast_block ? am : 1.0f);
            const float x_lo = fast_block ? am * kXRel : __builtin_inff();
            ok = mn >= x_lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float q0 = v[i] * r;
                const float e = __builtin_fmaf(-q0, am, v[i]);
                t[i] = __builtin_fmaf(e, r, q0);
            }
        }
        if (!ok) {
            const float a_div = am == 0.0f ? 1.0f : am;   // zero block: x is +-0, t = +-0
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = v[i] / a_div;
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

        if constexpr (!kTail) {
            *reinterpret_cast<uint32_t*>(codes + base / 2) = word;
            if ((lane % G) == 0) absmax[base / B] = am;
        } else {
            if (base < n) {
                if (base + 8 <= n) {
                    *reinterpret_cast<uint32_t*>(codes + base / 2) = word;
                } else {
                    // codes of elements past n are 0, bytes past ceil(n/2) are not written
                    const int64_t valid = n - base;          // 1..7
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int64_t e0 = 2 * j;
                        if (e0 >= valid) break;
                        uint32_t byte = (word >> (8 * j)) & 0xFFu;
                        if (e0 + 1 >= valid) byte &= 0xF0u;
                        codes[base / 2 + j] = (uint8_t)byte;
                    }
                }
                if ((lane % G) == 0) absmax[base / B] = am;
            }
        }
    };
    using Full = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;
    // The empty asm statements keep the loads of the other batch ahead of every use of
    // this one (the scheduler would otherwise move the unpacking up and wait for this
    // batch before the other one's loads are issued) ...
    auto pin = [](Raw (&rs)[kBatch]) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            Raw& r = rs[k];
            if constexpr (__is_same(InT, F32In)) {
                asm volatile("" : "+v"(r[0].x), "+v"(r[0].y), "+v"(r[0].z), "+v"(r[0].w),
                                  "+v"(r[1].x), "+v"(r[1].y), "+v"(r[1].z), "+v"(r[1].w) :: "memory");
            } else {
                asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w) :: "memory");
            }
        }
    };
    // ... and keep a batch's registers live past its stores, so that no store reads a
    // register that the next load into the same buffer overwrites (such a store would
    // have to complete first, and with it the other batch's loads).
    auto keep = [](const Raw (&rs)[kBatch]) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const Raw& r = rs[k];
            if constexpr (__is_same(InT, F32In)) {
                asm volatile("" :: "v"(r[0].x), "v"(r[0].y), "v"(r[0].z), "v"(r[0].w),
                                   "v"(r[1].x), "v"(r[1].y), "v"(r[1].z), "v"(r[1].w) : "memory");
            } else {
                asm volatile("" :: "v"(r.x), "v"(r.y), "v"(r.z), "v"(r.w) : "memory");
            }
        }
    };
    // Two batches in flight: a batch's buffer is reloaded (with the batch two turns
    // ahead) as soon as it has been processed, so every wait leaves the other buffer's
    // loads outstanding.  Batch b holds units b * kBatch + [0, kBatch).
    Raw ra[kBatch], rb[kBatch];
    int64_t b = wave;
    if (b < nbatches) {
        load_batch(b, ra);
        load_batch(b + nwaves, rb);
        for (;;) {
            pin(ra);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) process(b * kBatch + k, ra[k], Full{});
            keep(ra);
            if (b + nwaves >= nbatches) break;
            load_batch(b + 2 * nwaves, ra);
            pin(rb);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) process((b + nwaves) * kBatch + k, rb[k], Full{});
            keep(rb);
            b += 2 * nwaves;
            if (b >= nbatches) break;
            load_batch(b + nwaves, rb);
        }
    }
    // the units after the last full batch (fewer than kBatch full ones and the partial
    // last one), with per-element loads
    for (int64_t ut = nbatches * kBatch + wave; ut < nunits; ut += nwaves) {
        Raw r;
        load_raw<InT>(x, n, ut * kUnitElems + lane * 8, r);
        process(ut, r, Tail{});
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
    const int64_t waves_needed = nunits / kBatch > 0 ? nunits / kBatch : 1;
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
