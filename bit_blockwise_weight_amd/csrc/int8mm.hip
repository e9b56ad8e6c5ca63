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
// Matmul: 128 x 128 output tiles, 128 k per step, 4 waves as 2 x 2, each 64 x 64
// = 2 x 2 tiles of v_mfma_i32_32x32x32_i8 (exact int32 sums); both operands
// staged through double-buffered LDS with 128-byte rows whose 16-byte pieces are
// XOR-swizzled (piece c of row r in slot c ^ ((r >> 1) & 7): conflict-free
// fragment reads); the global loads run two steps ahead; one barrier per step.  Epilogue: C = RN(RN(float(acc) * SX[m])
// * SCB[n]) / 127^2 in fp32, then the outlier columns 16 at a time with
// v_mfma_f32_32x32x16_f16 into the same fp32 accumulators (X's fp16 values and the
// weight columns dequantized to fp16, CB * SCB / 127), fp16 output.
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
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
    using Raw = typename RawOf<InT>::type;
    for (int64_t row = wave; row < rows; row += nwaves) {
        const int64_t rbase = row * cols;
        float am = 0.0f;
        for (int64_t k = 8 * lane; k < cols; k += 512) {
            Raw r;
            load_raw<InT>(x, rbase + cols, rbase + k, r);
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
        for (int64_t k = 8 * lane; k < cols; k += 512) {
            Raw r;
            load_raw<InT>(x, rbase + cols, rbase + k, r);
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

// Column maxima of |x|: workgroup (bx, s) takes 512 columns (lane l: [512 bx + 8 l, + 8))
// and slice s of the rows, its 4 waves every 4th row of the slice; the 4 wave maxima
// meet in LDS and one atomicMax per column and slice goes to memory.  K % 8 == 0.
template <typename InT>
__global__ __launch_bounds__(kThreads) void colmax_kernel(const void* __restrict__ x, int64_t M, int64_t K,
                                                          int32_t nslices, uint32_t* __restrict__ colmax_bits) {
    __shared__ float part[3][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t k = 512 * (int64_t)blockIdx.x + 8 * lane;
    const bool ok = k < K;
    const int s = blockIdx.y;
    const int64_t r0 = M * s / nslices, r1 = M * (s + 1) / nslices;
    using Raw = typename RawOf<InT>::type;
    float mx[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
        for (int64_t m = r0 + wave; m < r1; m += 4) {
            Raw r;
            load_raw<InT>(x, (m + 1) * K, m * K + k, r);
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

constexpr int TM = 128, TN = 128, TKB = 128;
constexpr int kXcds = 8;

__device__ __forceinline__ int soff(int row, int chunk) { return row * 128 + 16 * (chunk ^ ((row >> 1) & 7)); }

__global__ __launch_bounds__(kThreads) void int8mm_kernel(MmArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t xa0[TM * TKB];
    __shared__ __attribute__((aligned(16))) int8_t xa1[TM * TKB];
    __shared__ __attribute__((aligned(16))) int8_t wb0[TN * TKB];
    __shared__ __attribute__((aligned(16))) int8_t wb1[TN * TKB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int fi = lane & 31, h = lane >> 5;
    const int64_t M = a.M, N = a.N, K = a.K;
    const uint32_t tiles_n = (uint32_t)((N + TN - 1) / TN);
    const uint32_t nt = (uint32_t)((M + TM - 1) / TM) * tiles_n;
    const uint32_t bid = blockIdx.x;
    const uint32_t lid = (nt % kXcds == 0) ? (bid % kXcds) * (nt / kXcds) + bid / kXcds : bid;
    const int64_t m0 = (int64_t)(lid / tiles_n) * TM, n0 = (int64_t)(lid % tiles_n) * TN;
    const int64_t nsteps = (K + TKB - 1) / TKB;

    // staging: piece c = tid + 256 v of a 128 x 128-byte tile: row c >> 3, 16-byte piece c & 7;
    // pieces at k >= K (the tail, and steps past the last) are zeros without a load
    auto load = [&](uint4 (&ra)[4], uint4 (&rb)[4], int64_t st) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = tid + kThreads * v;
            const int row = c >> 3, ch = c & 7;
            const int64_t k = st * TKB + 16 * ch;
            const int64_t gm = m0 + row < M ? m0 + row : M - 1;
            const int64_t gn = n0 + row < N ? n0 + row : N - 1;
            ra[v] = k < K ? *reinterpret_cast<const uint4*>(a.Xq + gm * K + k) : make_uint4(0, 0, 0, 0);
            rb[v] = k < K ? *reinterpret_cast<const uint4*>(a.CB + gn * K + k) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](const uint4 (&ra)[4], const uint4 (&rb)[4], int8_t* xa, int8_t* wb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = tid + kThreads * v;
            *reinterpret_cast<uint4*>(xa + soff(c >> 3, c & 7)) = ra[v];
            *reinterpret_cast<uint4*>(wb + soff(c >> 3, c & 7)) = rb[v];
        }
    };
    intx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    auto compute = [&](const int8_t* xa, const int8_t* wb) {
#pragma unroll
        for (int kk = 0; kk < TKB / 32; ++kk) {
            v4i_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const v4i_t*>(xa + soff(wm * 64 + 32 * i + fi, 2 * kk + h));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const v4i_t*>(wb + soff(wn * 64 + 32 * j + fi, 2 * kk + h));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // LDS stores done, loads in flight left alone
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // two register sets: the loads of step s + 2 are issued while step s is computed
    uint4 ra0[4], rb0[4], ra1[4], rb1[4];
    load(ra0, rb0, 0);
    store(ra0, rb0, xa0, wb0);
    load(ra1, rb1, 1);
    barrier();
    int64_t st = 0;
    for (; st + 1 < nsteps; st += 2) {
        load(ra0, rb0, st + 2);
        compute(xa0, wb0);
        store(ra1, rb1, xa1, wb1);
        barrier();
        load(ra1, rb1, st + 3);
        compute(xa1, wb1);
        store(ra0, rb0, xa0, wb0);
        barrier();
    }
    if (st < nsteps) compute(xa0, wb0);

    // epilogue: lane holds C[8 b + 4 h + q][fi] in register 4 b + q
    floatx16_t f[2][2];
    float scb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + 32 * j + fi;
        scb[j] = a.SCB[n < N ? n : N - 1];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t m = m0 + wm * 64 + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
            const float sx = a.SX[m < M ? m : M - 1];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                f[i][j][e] = __fdiv_rn(__fmul_rn(__fmul_rn((float)acc[i][j][e], sx), scb[j]), 16129.0f);
        }
    const int32_t nout = a.ocount ? *a.ocount : 0;
    for (int32_t c0 = 0; c0 < nout; c0 += 16) {
        halfx8_t xo[2], wo[2];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int32_t oi = c0 + 8 * h + p;
            const bool live = oi < nout;
            const int64_t col = live ? a.oidx[oi] : 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int64_t m = m0 + wm * 64 + 32 * i + fi;
                m = m < M ? m : M - 1;
                xo[i][p] = live ? a.X[m * K + col] : (_Float16)0.0f;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int64_t n = n0 + wn * 64 + 32 * j + fi;
                n = n < N ? n : N - 1;
                const float wd = __fdiv_rn(__fmul_rn((float)a.CB[n * K + col], scb[j]), 127.0f);
                wo[j][p] = live ? (_Float16)wd : (_Float16)0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) f[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xo[i], wo[j], f[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + fi;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 64 + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
                if (m < M && n < N) a.Y[m * N + n] = (_Float16)f[i][j][e];
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
    // about 512 workgroups, at least 64 rows per slice
    const int64_t colblocks = (K + 511) / 512;
    int64_t slices = (512 + colblocks - 1) / colblocks;
    if (slices > M / 64) slices = M / 64;
    if (slices < 1) slices = 1;
    if (slices > 65535) slices = 65535;
    hipLaunchKernelGGL((colmax_kernel<InT>), dim3((unsigned)colblocks, (unsigned)slices), dim3(kThreads), 0, s, x, M, K,
                       (int32_t)slices, colmax_bits);
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
    hipLaunchKernelGGL(int8mm_kernel, dim3((unsigned)nt), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qk
