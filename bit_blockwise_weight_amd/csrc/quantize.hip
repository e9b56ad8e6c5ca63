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
// Division.  For bf16 and fp16 inputs t = RN(x/a) is computed from one
// reciprocal per block, r = RN(1/a), and Markstein's correction
//     q0 = x*r,  e = fma(-q0, a, x),  t = fma(e, r, q0),
// which equals the IEEE quotient bit for bit whenever 2^-36 <= a <= 2^64 and
// |x| >= a*2^-64.  r itself is the hardware's approximate reciprocal y refined
// once, r = fma(fma(-a, y, 1), y, y).  Both steps are checked exhaustively over
// every bf16 and every fp16 value by the CPU test of the division (the
// reciprocal for every y within 2 ulp of 1/a).  Any lane holding an element
// outside that region redoes its 8 divisions with the IEEE sequence; fp32 inputs
// always use it.  When no decision threshold of the level table lies in
// (-2^-60, 2^-60] (FP4, whose levels include 0, is such a table; NF4, whose two
// middle levels are +-0.0396 with the threshold at the least positive float, is
// not), the condition on |x| is dropped: an x with |x| < a*2^-64 has |x/a| < 2^-64
// and a computed t below 2^-60 in magnitude, and every t in that range gets the
// same code.
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
constexpr int kMaxQuantGroup = 16;        // arrays per launch
// a tensor of this many elements or more is quantized in a launch of its own: measured on
// a 70B-shaped layer (67 M to 235 M elements per weight), seven single launches took
// 515-550 us and one grouped launch 566-572 us, while the seven Llama-7B weights (17 M
// and 45 M) took 125 us as single launches and 95 us grouped
constexpr int64_t kQuantAloneElems = (int64_t)1 << 26;

constexpr float kAMin = 0x1p-36f;
constexpr float kAMax = 0x1p64f;
constexpr float kXRel = 0x1p-64f;

// The arrays of one launch (a single call is a group of one): array t owns the global
// batches [batch0[t], batch0[t + 1]) and the global tail units [tail0[t], tail0[t + 1])
// (a launch holds fewer than 2^30 batches).
struct QuantArray {
    const void* x;
    int64_t n;
    uint8_t* codes;
    float* absmax;
};
struct QuantGroup {
    QuantArray a[kMaxQuantGroup];
    int32_t batch0[kMaxQuantGroup + 1];
    int32_t tail0[kMaxQuantGroup + 1];
    int32_t count;
};

template <typename InT, int B, bool kSorted, bool kTinyFree>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(QuantGroup g, QuantLut lut) {
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
    // uniform in the wave: the loop below is then scalar control flow
    const int64_t wave = (int64_t)blockIdx.x * (kQThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kQThreads / kWave);
    const char* lds_bytes = reinterpret_cast<const char*>(lut_lds);

    const int64_t nbatches = g.batch0[g.count];     // batches of kBatch full units, all arrays
    // the array of the next batch loaded, the first batch of the array after it and the
    // array's pointers: a wave loads its batches in increasing order, so the cursor only
    // moves forward, and the descriptor is read only when it crosses into the next array
    // (one scalar compare per batch otherwise; no scalar load in front of a batch's loads)
    int tl = 0;
    int32_t tl_start = 0;
    int32_t tl_end = g.count > 1 ? g.batch0[1] : INT32_MAX;
    QuantArray cur = g.a[0];

    using Raw = typename RawOf<InT>::type;
    // where a loaded batch belongs: its array and the array's first unit of the batch
    struct Place {
        QuantArray arr;
        int64_t unit;
    };
    // A batch: one unconditional load per lane and unit (the batch index is clamped, so
    // the prefetch past the last batch re-reads it); no branch separates a load from
    // the code that waits for it, so the other batch's loads stay in flight meanwhile.
    auto load_batch = [&](int64_t bi, Raw (&r)[kBatch]) {
        const int32_t bc = (int32_t)(bi < nbatches ? bi : nbatches - 1);
        while (bc >= tl_end) {
            ++tl;
            tl_start = tl_end;
            tl_end = tl + 1 < g.count ? g.batch0[tl + 1] : INT32_MAX;
            cur = g.a[tl];
        }
        const int64_t u0 = (int64_t)(bc - tl_start) * kBatch;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) load_raw_full<InT>(cur.x, (u0 + k) * kUnitElems + lane * 8, r[k]);
        return Place{cur, u0};
    };
    auto process = [&](const QuantArray& arr, int64_t unit, const Raw& raw, auto tail_tag) {
        const int64_t n = arr.n;
        uint8_t* __restrict__ codes = arr.codes;
        float* __restrict__ absmax = arr.absmax;
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
            // am is a non-negative float (or NaN, above the range), so its bit pattern
            // orders like its value
            const bool fast_block = as_uint(am) - as_uint(kAMin) <= as_uint(kAMax) - as_uint(kAMin);
            // RN(1/a): the hardware reciprocal (within 1 ulp) and one correction step,
            // exact for every bf16 and fp16 a of the fast region (CPU-checked, with a 2 ulp
            // margin on the hardware's error).  Outside the region t is recomputed below.
            const float r0 = __builtin_amdgcn_rcpf(am);
            const float r = __builtin_fmaf(__builtin_fmaf(-am, r0, 1.0f), r0, r0);
            if constexpr (kTinyFree) ok = fast_block;
            else ok = fast_block && mn >= am * kXRel;
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
            if constexpr (kFastDiv) {
                // finite input gives |t| <= 1; a non-finite block (outside the contract) is
                // the only way here to anything else, and it maps to 0, so the table read
                // below needs no clamp (the fast path never sees a non-finite absmax)
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = __builtin_fabsf(t[i]) <= 1.0f ? t[i] : 0.0f;
            }
        }

        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // |t| <= 1 gives the pattern 0x4B000000 + bin, bin in [0, 2S]; for fp32 input the
            // min keeps a non-finite t (outside the contract) inside the table
            uint32_t bin = as_uint(__builtin_fmaf(t[i], S, C));
            if constexpr (!kFastDiv) bin = min(bin, bin_cap);
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
            // the unit's bases are uniform: the stores take a scalar base and a lane offset
            uint8_t* cu = codes + unit * (kUnitElems / 2);
            float* au = absmax + unit * (kUnitElems / B);
            *reinterpret_cast<uint32_t*>(cu + 4 * lane) = word;
            if ((lane % G) == 0) au[lane / G] = am;
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
        Place pa = load_batch(b, ra);
        Place pb = load_batch(b + nwaves, rb);
        for (;;) {
            pin(ra);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) process(pa.arr, pa.unit + k, ra[k], Full{});
            keep(ra);
            if (b + nwaves >= nbatches) break;
            pa = load_batch(b + 2 * nwaves, ra);
            pin(rb);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) process(pb.arr, pb.unit + k, rb[k], Full{});
            keep(rb);
            b += 2 * nwaves;
            if (b >= nbatches) break;
            pb = load_batch(b + nwaves, rb);
        }
    }
    // each array's units after its last full batch (fewer than kBatch full ones and the
    // partial last one), with per-element loads
    const int32_t ntails = g.tail0[g.count];
    int tt = 0;
    for (int32_t gt = (int32_t)wave; gt < ntails; gt += (int32_t)nwaves) {
        while (tt + 1 < g.count && gt >= g.tail0[tt + 1]) ++tt;
        const QuantArray& arr = g.a[tt];
        const int64_t ut = (int64_t)(g.batch0[tt + 1] - g.batch0[tt]) * kBatch + (gt - g.tail0[tt]);
        Raw r;
        load_raw<InT>(arr.x, arr.n, ut * kUnitElems + lane * 8, r);
        process(arr, ut, r, Tail{});
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
hipError_t launch_typed(const QuantGroup& g, int64_t nunits_total, const QuantLut& lut, hipStream_t s) {
    const int64_t waves_needed = nunits_total / kBatch > 0 ? nunits_total / kBatch : 1;
    const int64_t wgs_needed = (waves_needed + (kQThreads / kWave) - 1) / (kQThreads / kWave);
    const int64_t cap = (int64_t)num_cus() * kWgsPerCu;   // persistent: the LDS table is filled once per workgroup
    const int grid = (int)(wgs_needed < cap ? wgs_needed : cap);
    const size_t lds = (size_t)lut.nbins * kLutCopies * sizeof(uint2);
    // the condition on small |x| only exists for the reciprocal division of 16-bit input
    const bool tiny_free = lut.tiny_free != 0 && !__is_same(InT, F32In);
    if (lut.sorted) {
        if (tiny_free) hipLaunchKernelGGL((quantize_kernel<InT, B, true, true>), dim3(grid), dim3(kQThreads), lds, s, g, lut);
        else hipLaunchKernelGGL((quantize_kernel<InT, B, true, false>), dim3(grid), dim3(kQThreads), lds, s, g, lut);
    } else {
        if (tiny_free) hipLaunchKernelGGL((quantize_kernel<InT, B, false, true>), dim3(grid), dim3(kQThreads), lds, s, g, lut);
        else hipLaunchKernelGGL((quantize_kernel<InT, B, false, false>), dim3(grid), dim3(kQThreads), lds, s, g, lut);
    }
    return hipGetLastError();
}

template <typename InT>
hipError_t launch_bs(const QuantGroup& g, int64_t nunits_total, int32_t blocksize, const QuantLut& lut,
                     hipStream_t s) {
    switch (blocksize) {
        case 64: return launch_typed<InT, 64>(g, nunits_total, lut, s);
        case 128: return launch_typed<InT, 128>(g, nunits_total, lut, s);
        case 256: return launch_typed<InT, 256>(g, nunits_total, lut, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_group(const QuantGroup& g, int64_t nunits_total, int32_t x_dtype, int32_t blocksize,
                        const QuantLut& lut, hipStream_t s) {
    switch (x_dtype) {
        case QK_BF16: return launch_bs<Bf16In>(g, nunits_total, blocksize, lut, s);
        case QK_F16: return launch_bs<F16In>(g, nunits_total, blocksize, lut, s);
        case QK_F32: return launch_bs<F32In>(g, nunits_total, blocksize, lut, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int device_cu_count() { return num_cus(); }

hipError_t launch_quantize_group(const QuantItem* items, int32_t count, int32_t x_dtype, int32_t blocksize,
                                 const QuantLut& lut, hipStream_t s) {
    QuantGroup g;
    int64_t nunits_total = 0;
    auto flush = [&]() -> hipError_t {
        if (g.count == 0) return hipSuccess;
        const hipError_t e = launch_group(g, nunits_total, x_dtype, blocksize, lut, s);
        g.count = 0;
        nunits_total = 0;
        return e;
    };
    g.count = 0;
    g.batch0[0] = 0;
    g.tail0[0] = 0;
    for (int32_t i = 0; i < count; ++i) {
        const QuantItem& it = items[i];
        const int64_t nunits = (it.n + kUnitElems - 1) / kUnitElems;
        const int64_t nbatches = it.n / kUnitElems / kBatch;
        if (it.n >= kQuantAloneElems && g.count > 0) {
            const hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        // a launch holds at most kMaxQuantGroup arrays and fewer than 2^30 batches and
        // tail units (32-bit prefix tables; one array of the library's sizes fits)
        if (g.count == kMaxQuantGroup || (g.count > 0 && (int64_t)g.batch0[g.count] + nbatches >= ((int64_t)1 << 30))) {
            const hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        const int t = g.count;
        g.a[t] = QuantArray{it.x, it.n, it.codes, it.absmax};
        g.batch0[t + 1] = g.batch0[t] + (int32_t)nbatches;
        g.tail0[t + 1] = g.tail0[t] + (int32_t)(nunits - nbatches * kBatch);
        g.count = t + 1;
        nunits_total += nunits;
        if (it.n >= kQuantAloneElems) {
            const hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
    }
    return flush();
}

hipError_t launch_quantize(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize, const QuantLut& lut,
                           uint8_t* codes, float* absmax, hipStream_t s) {
    const QuantItem it{x, n, codes, absmax};
    return launch_quantize_group(&it, 1, x_dtype, blocksize, lut, s);
}

}  // namespace qk
