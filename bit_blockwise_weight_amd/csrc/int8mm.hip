// LLM.int8(): row-wise int8 quantization, outlier columns, and the int8 matmul
// with the 16-bit outlier product fused into its epilogue, for gfx950.
//
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.1 LLM.int8(), 【原理】, 【代码】,
// 【例子】 and figure 2-1: the activation columns whose largest magnitude exceeds
// the threshold are outlier features and take a 16-bit matmul with the matching
// weight columns; every other column is quantized vector-wise (one absmax per row,
// values scaled to [-127, 127], int8) and multiplied with the int8 weight (one
// absmax per weight row); the two results are added.  Threshold 0 disables the
// decomposition.
//
// Quantization of a row with absmax a: q = rint(RN(RN(x / a) * 127)) (IEEE
// division, round half to even), 0 when a == 0 or the column is excluded.
//
// Outlier columns: column maxima reduced inside a workgroup, then by atomicMax on
// the bits of non-negative floats across row slices (the maximum does not depend
// on the order), then one workgroup lists the columns over the threshold in
// increasing order (a prefix sum, deterministic).
//
// Matmul: 256 x 256 output tiles, 64 k per step, 8 waves as 4 x 2, each 64 x 128
// = 2 x 4 tiles of v_mfma_i32_32x32x32_i8 (exact int32 sums; 6 fragment reads per
// 8 MFMAs; two waves per SIMD); both operands staged through double-buffered LDS with 64-byte rows
// whose 16-byte pieces are XOR-swizzled (conflict-free fragment reads); the global
// loads run two steps ahead; one barrier per step.  Epilogue: C = RN(RN(float(acc) * SX[m])
// * SCB[n]) / 127^2 in fp32, plus the outlier columns' product computed with
// v_mfma_f32_32x32x16_f16 from X's fp16 values and the weight columns dequantized
// to fp16 (CB * SCB / 127), gathered by the workgroup into LDS; fp16 output, each
// 32 x 32 tile passed through a wave-private LDS area so it leaves in 16-byte stores.
#include "qk_internal.h"
#include "qk_device.h"
#include "qk_quant_io.h"

namespace qk {
namespace {

typedef int intx16_t __attribute__((ext_vector_type(16)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max64(float v) {
    v = group_max<32>(v);
    return fmaxf(as_float(__builtin_amdgcn_readlane(as_uint(v), 0)), as_float(__builtin_amdgcn_readlane(as_uint(v), 32)));
}

// 8 elements at element offset e (in range, 16-byte aligned): one 16-byte load for
// 16-bit types, two for fp32, without the tail handling of load_raw
template <typename InT>
__device__ __forceinline__ void load8(const void* x, int64_t e, typename RawOf<InT>::type& r) {
    if constexpr (__is_same(InT, F32In)) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + e);
        r[0] = p[0];
        r[1] = p[1];
    } else {
        r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + e);
    }
}

__device__ __forceinline__ int32_t quant127(float x, float a) {
    if (a == 0.0f) return 0;
    return (int32_t)__builtin_rintf(__fmul_rn(x / a, 127.0f));
}

// One wave per row (grid-stride over rows); lane l takes columns [512 i + 8 l, + 8).
// cols % 8 == 0.  skip: 1 byte per column, non-zero = excluded (or null).
template <typename InT>
__global__ __launch_bounds__(kThreads) void rowquant_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                            const uint8_t* __restrict__ skip, int8_t* __restrict__ q,
                                                            float* __restrict__ absmax) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
    using Raw = typename RawOf<InT>::type;
    for (int64_t row = wave; row < rows; row += nwaves) {
        const int64_t rbase = row * cols;
        float am = 0.0f;
#pragma unroll 4
        for (int64_t k = 8 * lane; k < cols; k += 512) {
            Raw r;
            load8<InT>(x, rbase + k, r);
            float v[8];
            unpack_raw<InT>(r, v);
            uint2 sk = make_uint2(0u, 0u);
            if (skip) sk = *reinterpret_cast<const uint2*>(skip + k);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t s = ((i < 4 ? sk.x : sk.y) >> (8 * (i & 3))) & 0xFFu;
                am = s ? am : fmaxf(am, fabsf(v[i]));
            }
        }
        am = wave_max64(am);
#pragma unroll 4
        for (int64_t k = 8 * lane; k < cols; k += 512) {
            Raw r;
            load8<InT>(x, rbase + k, r);
            float v[8];
            unpack_raw<InT>(r, v);
            uint2 sk = make_uint2(0u, 0u);
            if (skip) sk = *reinterpret_cast<const uint2*>(skip + k);
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t s = ((i < 4 ? sk.x : sk.y) >> (8 * (i & 3))) & 0xFFu;
                const int32_t qi = s ? 0 : quant127(v[i], am);
                w[i >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (i & 3));
            }
            *reinterpret_cast<uint2*>(q + rbase + k) = make_uint2(w[0], w[1]);
        }
        if (lane == 0) absmax[row] = am;
    }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Column maxima of |x|: a workgroup takes 512 columns (lane l: [512 c + 8 l, + 8)) and
// one slice of the rows, its 4 waves every 4th row of the slice; the 4 wave maxima
// meet in LDS and one atomicMax per column and slice goes to memory.  All slices of
// a column block run on one XCD (workgroup i runs on XCD i % 8), so the atomics on a
// column stay in that XCD's L2.  K % 8 == 0.
template <typename InT>
__global__ __launch_bounds__(kThreads) void colmax_kernel(const void* __restrict__ x, int64_t M, int64_t K,
                                                          int32_t nslices, uint32_t* __restrict__ colmax_bits) {
    __shared__ float part[3][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t ncb = (K + 511) / 512;
    const int64_t xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int64_t cb = xcd + 8 * (idx / nslices);            // column block, on XCD cb % 8
    const int s = (int)(idx % nslices);
    if (cb >= ncb) return;
    const int64_t k = 512 * cb + 8 * lane;
    const bool ok = k < K;
    const int64_t r0 = M * s / nslices, r1 = M * (s + 1) / nslices;
    using Raw = typename RawOf<InT>::type;
    float mx[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
#pragma unroll 8
        for (int64_t m = r0 + wave; m < r1; m += 4) {
            Raw r;
            load8<InT>(x, m * K + k, r);
            float v[8];
            unpack_raw<InT>(r, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(v[i]));
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) part[wave - 1][8 * lane + i] = mx[i];
    }
    __syncthreads();
    if (wave == 0 && ok && r1 > r0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float m4 = fmaxf(fmaxf(mx[i], part[0][8 * lane + i]), fmaxf(part[1][8 * lane + i], part[2][8 * lane + i]));
            atomicMax(colmax_bits + k + i, as_uint(m4));   // non-negative: bit order = value order
        }
    }
}

// One workgroup of 1024 threads: flags[k] = colmax[k] > threshold (threshold > 0),
// idx = the flagged columns in increasing order, count[0] = how many.
__global__ __launch_bounds__(1024) void outlier_list_kernel(const uint32_t* __restrict__ colmax_bits, int64_t K,
                                                            float threshold, uint8_t* __restrict__ flags,
                                                            int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    const int64_t per = (K + 1023) / 1024;
    const int64_t c0 = t * per, c1 = (c0 + per < K) ? c0 + per : K;
    const bool on = threshold > 0.0f;
    int32_t local = 0;
    for (int64_t c = c0; c < c1; ++c) local += (on && as_float(colmax_bits[c]) > threshold) ? 1 : 0;
    part[t] = local;
    __syncthreads();
    // inclusive scan (Hillis-Steele)
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int32_t pos = part[t] - local;
    for (int64_t c = c0; c < c1; ++c) {
        const bool o = on && as_float(colmax_bits[c]) > threshold;
        flags[c] = o ? 1 : 0;
        if (o) idx[pos++] = (int32_t)c;
    }
    if (t == 1023) count[0] = part[1023];
}

struct MmArgs {
    const int8_t* Xq;      // [M, K]
    const float* SX;       // [M]
    const int8_t* CB;      // [N, K]
    const float* SCB;      // [N]
    const _Float16* X;     // [M, K] fp16 (outlier source) or null
    const int32_t* oidx;   // outlier columns, increasing
    const int32_t* ocount; // device scalar
    _Float16* Y;           // [M, N]
    int64_t M, N, K;
};

constexpr int TM = 256, TN = 256, TKB = 64;
constexpr int kXcds = 8;
constexpr int kOGroup = 32;                 // outlier columns staged at a time (2 MFMA steps of 16)
constexpr int kOPitch = kOGroup + 8;        // fp16 per staged outlier row (80 bytes: conflict-free reads)

// byte offset of 16-byte piece c of row r in a tile of 64-byte rows: piece c sits in
// slot c ^ ((r >> 2) & 3), so 16 consecutive rows reading one piece hit 16 bank groups
__device__ __forceinline__ int soff(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 2) & 3)); }

constexpr int kMmThreads = 512;            // 8 waves: two per SIMD, so one wave's MFMAs cover the other's waits

template <bool kTail>
__global__ __launch_bounds__(kMmThreads, 1) void int8mm_kernel(MmArgs a) {
    // one pool: X tiles at 0 and 16 KB, W tiles at 32 and 48 KB; the epilogue reuses it
    // for the staged outlier columns (X part at 0, W part at 32 KB, 20 KB each)
    __shared__ __attribute__((aligned(16))) int8_t pool[2 * TM * TKB + 2 * TN * TKB];
    int8_t* const xa0 = pool;
    int8_t* const xa1 = pool + TM * TKB;
    int8_t* const wb0 = pool + 2 * TM * TKB;
    int8_t* const wb1 = pool + 2 * TM * TKB + TN * TKB;
    static_assert(TM * kOPitch * 2 <= 2 * TM * TKB && TN * kOPitch * 2 <= 2 * TN * TKB, "outlier staging fits");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;                     // wave tile: rows [64 wm, +64) x cols [128 wn, +128)
    const int fi = lane & 31, h = lane >> 5;
    const int64_t M = a.M, N = a.N, K = a.K;
    const uint32_t tiles_n = (uint32_t)((N + TN - 1) / TN);
    const uint32_t nt = (uint32_t)((M + TM - 1) / TM) * tiles_n;
    const uint32_t bid = blockIdx.x;
    const uint32_t lid = (nt % kXcds == 0) ? (bid % kXcds) * (nt / kXcds) + bid / kXcds : bid;
    const int64_t m0 = (int64_t)(lid / tiles_n) * TM, n0 = (int64_t)(lid % tiles_n) * TN;
    const int64_t nsteps = (K + TKB - 1) / TKB;

    // staging: piece c = tid + 512 v (v < 2) of a 256 x 64-byte tile: row c >> 2, piece c & 3
    const int8_t* xrow[2];
    const int8_t* wrow[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int row = (tid + kMmThreads * v) >> 2;
        const int64_t gm = m0 + row < M ? m0 + row : M - 1;
        const int64_t gn = n0 + row < N ? n0 + row : N - 1;
        xrow[v] = a.Xq + gm * K;
        wrow[v] = a.CB + gn * K;
    }
    // unconditional loads from a clamped address (a conditional load would become a
    // branch); with K % 64 != 0 the pieces at k >= K of the last step are zeroed when
    // they are stored.  Steps past the last are loaded (clamped) but never computed.
    auto load = [&](uint4 (&ra)[2], uint4 (&rb)[2], int64_t st) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int64_t k = st * TKB + 16 * ((tid + kMmThreads * v) & 3);
            const int64_t kc = k < K ? k : K - 16;
            ra[v] = *reinterpret_cast<const uint4*>(xrow[v] + kc);
            rb[v] = *reinterpret_cast<const uint4*>(wrow[v] + kc);
        }
    };
    auto store = [&](const uint4 (&ra)[2], const uint4 (&rb)[2], int64_t st, int8_t* xa, int8_t* wb) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int c = tid + kMmThreads * v;
            uint4 va = ra[v], vb = rb[v];
            if constexpr (kTail) {
                const bool kin = st * TKB + 16 * (c & 3) < K;
                va = make_uint4(kin ? va.x : 0u, kin ? va.y : 0u, kin ? va.z : 0u, kin ? va.w : 0u);
                vb = make_uint4(kin ? vb.x : 0u, kin ? vb.y : 0u, kin ? vb.z : 0u, kin ? vb.w : 0u);
            }
            *reinterpret_cast<uint4*>(xa + soff(c >> 2, c & 3)) = va;
            *reinterpret_cast<uint4*>(wb + soff(c >> 2, c & 3)) = vb;
        }
    };
    intx16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    auto compute = [&](const int8_t* xa, const int8_t* wb) {
#pragma unroll
        for (int kk = 0; kk < TKB / 32; ++kk) {
            v4i_t af[2], bf[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const v4i_t*>(xa + soff(wm * 64 + 32 * i + fi, 2 * kk + h));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const v4i_t*>(wb + soff(wn * 128 + 32 * j + fi, 2 * kk + h));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // LDS stores done, loads in flight left alone
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // two register sets: the loads of step s + 2 are issued while step s is computed;
    // the empty asm statements keep the scheduler from sinking the loads to the end of
    // the step (next to the stores that consume the other register set)
    uint4 ra0[2], rb0[2], ra1[2], rb1[2];
    load(ra0, rb0, 0);
    store(ra0, rb0, 0, xa0, wb0);
    load(ra1, rb1, 1);
    barrier();
    int64_t st = 0;
    for (; st + 1 < nsteps; st += 2) {
        load(ra0, rb0, st + 2);
        asm volatile("" ::: "memory");
        compute(xa0, wb0);
        store(ra1, rb1, st + 1, xa1, wb1);
        barrier();
        load(ra1, rb1, st + 3);
        asm volatile("" ::: "memory");
        compute(xa1, wb1);
        store(ra0, rb0, st + 2, xa0, wb0);
        barrier();
    }
    if (st < nsteps) compute(xa0, wb0);
    __syncthreads();

    // epilogue.  The outlier columns are staged in groups of 32: threads 0..255 take row
    // t of the tile's X columns (fp16), threads 256..511 row t - 256 of the weight
    // columns (CB * SCB / 127 in fp16), in LDS freed by the main loop.  Then tile by
    // tile: the outlier product in fp32 (v_mfma_f32_32x32x16_f16, 16 columns per MFMA),
    // plus the int32 sums scaled by SX[m] SCB[n] / 127^2, to fp16.  With more than 32
    // outlier columns every tile restages the groups (rare: the page's figure is 0.1%
    // of the columns).
    const int32_t nout = a.ocount ? *a.ocount : 0;
    const int ngroups = (nout + kOGroup - 1) / kOGroup;
    _Float16* xo = reinterpret_cast<_Float16*>(xa0);              // [TM][kOPitch] over xa0, xa1
    _Float16* wo = reinterpret_cast<_Float16*>(wb0);              // [TN][kOPitch] over wb0, wb1
    auto stage = [&](int g) {
        const int r = tid & 255;
        const bool xside = tid < 256;
        const int64_t m = m0 + r < M ? m0 + r : M - 1;
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        const float sn = a.SCB[n];
#pragma unroll 4
        for (int p = 0; p < kOGroup; ++p) {
            const int32_t oi = kOGroup * g + p;
            const bool live = oi < nout;
            const int64_t col = live ? a.oidx[oi] : 0;
            if (xside) xo[r * kOPitch + p] = live ? a.X[m * K + col] : (_Float16)0.0f;
            else wo[r * kOPitch + p] =
                live ? (_Float16)__fdiv_rn(__fmul_rn((float)a.CB[n * K + col], sn), 127.0f) : (_Float16)0.0f;
        }
    };
    if (ngroups == 1) {
        stage(0);
        __syncthreads();
    }
    const int64_t mrow = m0 + wm * 64 + 4 * h;                   // + 32 i + 8 b + q
    // a 2 KB LDS area per wave for the output tile, outside the staged outlier columns
    // (X part [0, 20 KB), W part [32, 52) KB): waves 0-5 at 20 KB + 2 KB w, 6-7 at 52 KB +
    uint16_t* yst = reinterpret_cast<uint16_t*>(pool + (wave < 6 ? 20480 + 2048 * wave : 53248 + 2048 * (wave - 6)));
    const bool vec_ok = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(a.Y) % 16) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            floatx16_t t;
#pragma unroll
            for (int e = 0; e < 16; ++e) t[e] = 0.0f;
            for (int g = 0; g < ngroups; ++g) {
                if (ngroups > 1) {
                    __syncthreads();
                    stage(g);
                    __syncthreads();
                }
#pragma unroll
                for (int c = 0; c < kOGroup / 16; ++c) {
                    const halfx8_t xf =
                        *reinterpret_cast<const halfx8_t*>(xo + (wm * 64 + 32 * i + fi) * kOPitch + 16 * c + 8 * h);
                    const halfx8_t wf =
                        *reinterpret_cast<const halfx8_t*>(wo + (wn * 128 + 32 * j + fi) * kOPitch + 16 * c + 8 * h);
                    t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf, wf, t, 0, 0, 0);
                }
            }
            const int64_t n = n0 + wn * 128 + 32 * j + fi;
            const float sn = a.SCB[n < N ? n : N - 1];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = mrow + 32 * i + 8 * (e / 4) + (e % 4);
                const float sx = a.SX[m < M ? m : M - 1];
                const float y = __fdiv_rn(__fmul_rn(__fmul_rn((float)acc[i][j][e], sx), sn), 16129.0f) + t[e];
                yst[(8 * (e / 4) + 4 * h + (e % 4)) * 32 + fi] = __builtin_bit_cast(uint16_t, (_Float16)y);
            }
            // the 32 x 32 tile back from the wave's LDS area, 16 bytes per lane: two
            // stores, each 16 rows x 64 contiguous bytes
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int row = 16 * half + (lane >> 2), q = lane & 3;
                const uint4 v = *reinterpret_cast<const uint4*>(yst + row * 32 + 8 * q);
                const int64_t gm = m0 + wm * 64 + 32 * i + row;
                const int64_t gn = n0 + wn * 128 + 32 * j + 8 * q;
                if (gm >= M || gn >= N) continue;
                uint16_t* dst = reinterpret_cast<uint16_t*>(a.Y) + gm * N + gn;
                if (vec_ok && gn + 8 <= N) {
                    *reinterpret_cast<uint4*>(dst) = v;
                } else {
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                    for (int t8 = 0; t8 < 8 && gn + t8 < N; ++t8) dst[t8] = (uint16_t)(w4[t8 >> 1] >> ((t8 & 1) ? 16 : 0));
                }
            }
        }
    }
}

template <typename InT>
hipError_t launch_rowquant_t(const void* x, int64_t rows, int64_t cols, const uint8_t* skip, int8_t* q,
                             float* absmax, hipStream_t s) {
    const int64_t wgs = (rows + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    hipLaunchKernelGGL((rowquant_kernel<InT>), dim3((unsigned)(wgs < cap ? wgs : cap)), dim3(kThreads), 0, s, x, rows,
                       cols, skip, q, absmax);
    return hipGetLastError();
}

template <typename InT>
hipError_t launch_colmax_t(const void* x, int64_t M, int64_t K, uint32_t* colmax_bits, hipStream_t s) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((K + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       colmax_bits, K);
    // about 512 workgroups, at least 64 rows per slice; column block c on XCD c % 8
    const int64_t colblocks = (K + 511) / 512;
    int64_t slices = (512 + colblocks - 1) / colblocks;
    if (slices > M / 64) slices = M / 64;
    if (slices < 1) slices = 1;
    const int64_t per_xcd = (colblocks + 7) / 8;
    const int64_t grid = 8 * per_xcd * slices;
    hipLaunchKernelGGL((colmax_kernel<InT>), dim3((unsigned)grid), dim3(kThreads), 0, s, x, M, K, (int32_t)slices,
                       colmax_bits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_int8_rowquant(const void* x, int32_t dtype, int64_t rows, int64_t cols, const uint8_t* skip,
                                int8_t* q, float* absmax, hipStream_t s) {
    switch (dtype) {
        case QK_BF16: return launch_rowquant_t<Bf16In>(x, rows, cols, skip, q, absmax, s);
        case QK_F16: return launch_rowquant_t<F16In>(x, rows, cols, skip, q, absmax, s);
        case QK_F32: return launch_rowquant_t<F32In>(x, rows, cols, skip, q, absmax, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_int8_outliers(const void* x, int32_t dtype, int64_t M, int64_t K, float threshold, float* colmax,
                                uint8_t* flags, int32_t* idx, int32_t* count, hipStream_t s) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(colmax);
    hipError_t e;
    switch (dtype) {
        case QK_BF16: e = launch_colmax_t<Bf16In>(x, M, K, bits, s); break;
        case QK_F16: e = launch_colmax_t<F16In>(x, M, K, bits, s); break;
        case QK_F32: e = launch_colmax_t<F32In>(x, M, K, bits, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(outlier_list_kernel, dim3(1), dim3(1024), 0, s, bits, K, threshold, flags, idx, count);
    return hipGetLastError();
}

hipError_t launch_int8_matmul(const int8_t* Xq, const float* SX, const int8_t* CB, const float* SCB, int64_t M,
                              int64_t N, int64_t K, const void* X, const int32_t* oidx, const int32_t* ocount, void* Y,
                              hipStream_t s) {
    MmArgs a;
    a.Xq = Xq; a.SX = SX; a.CB = CB; a.SCB = SCB;
    a.X = reinterpret_cast<const _Float16*>(X);
    a.oidx = oidx; a.ocount = ocount;
    a.Y = reinterpret_cast<_Float16*>(Y);
    a.M = M; a.N = N; a.K = K;
    const int64_t nt = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    if (nt > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (K % TKB == 0) hipLaunchKernelGGL((int8mm_kernel<false>), dim3((unsigned)nt), dim3(kMmThreads), 0, s, a);
    else hipLaunchKernelGGL((int8mm_kernel<true>), dim3((unsigned)nt), dim3(kMmThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qk
