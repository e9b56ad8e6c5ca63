// Double quantization of the absmax array for gfx950.
//
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 QLoRA / NF4, 【原理】② and
// 【代码】: the per-block absmax values are quantized again to 8 bits (state2),
// with an offset (read as their mean) subtracted first.  Definition used:
//     mean = RN_fp32(T / nb), T the fp64 sum along a perfect binary tree over the
//            absmax array zero-padded to a power of two (divided in fp64);
//     c_j  = RN_fp32(a_j - mean);  per block d of 256: s_d = max |c_j|,
//     scale_d = RN_fp32(s_d / 127), q_j = rint_even(RN_fp32(RN_fp32(c_j / s_d) * 127))
//     (q_j = 0 when s_d = 0).
//
// Kernels.
//   tree_partials: each workgroup sums an aligned chunk of 4096 values (fp32
//     absmax or fp64 partials) along the binary tree: every thread reduces 16
//     neighbours pairwise, then lanes combine with xor-butterflies (which add
//     exactly the tree's left and right subtrees), then the 4 waves pairwise.
//     Applied until at most 4096 partials remain.  An aligned chunk of a
//     power-of-two size is a subtree of the global tree, so the result is the
//     tree sum bit for bit.
//   dq_quantize: every workgroup first re-derives the mean from the final
//     partials (the same tree, at most 32 KB read from L2), then each wave
//     quantizes one block of 256 absmax (4 per lane).
#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

constexpr int kChunk = 4096;       // values per partial
constexpr int kThreads = 256;
constexpr int kPerThread = kChunk / kThreads;   // 16

__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// Tree sum of 16 register values (already in order) -> one double.
__device__ __forceinline__ double tree16(double (&a)[kPerThread]) {
#pragma unroll
    for (int w = kPerThread / 2; w >= 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    }
    return a[0];
}

// Sum of the 4096-value chunk held 16 per thread, in tree order; valid in thread 0.
__device__ __forceinline__ double chunk_tree(double (&a)[kPerThread], double* red) {
    double v = tree16(a);
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = v + shfl_xor_d(v, m);
    const int wv = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[wv] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void tree_partials(const T* __restrict__ in, int64_t count,
                                                          double* __restrict__ out) {
    __shared__ double red[kThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kChunk + (int64_t)threadIdx.x * kPerThread;
    double a[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) a[i] = (base + i < count) ? (double)in[base + i] : 0.0;
    const double s = chunk_tree(a, red);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

constexpr int kDqBlock = QK_DQ_BLOCK;           // 256 absmax per scale
constexpr int kDqBlocksPerWg = kThreads / kWave; // one block per wave

__global__ __launch_bounds__(kThreads) void dq_quantize(const float* __restrict__ absmax, int64_t nb,
                                                        const double* __restrict__ partials, int64_t npart,
                                                        int8_t* __restrict__ q8, float* __restrict__ scale,
                                                        float* __restrict__ mean_out) {
    __shared__ double red[kThreads / kWave];
    __shared__ float mean_sh;
    // mean from the final partials (npart <= 4096), same tree as the partial kernel
    {
        const int64_t base = (int64_t)threadIdx.x * kPerThread;
        double a[kPerThread];
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) a[i] = (base + i < npart) ? partials[base + i] : 0.0;
        const double total = chunk_tree(a, red);
        if (threadIdx.x == 0) {
            const float mu = (float)(total / (double)nb);
            mean_sh = mu;
            if (blockIdx.x == 0) *mean_out = mu;
        }
        __syncthreads();
    }
    const float mu = mean_sh;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t d = (int64_t)blockIdx.x * kDqBlocksPerWg + threadIdx.x / kWave;
    const int64_t nd = (nb + kDqBlock - 1) / kDqBlock;
    if (d >= nd) return;
    const int64_t base = d * kDqBlock + lane * 4;
    float c[4];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i] = (base + i < nb) ? __fsub_rn(absmax[base + i], mu) : 0.0f;
        m = fmaxf(m, fabsf(c[i]));
    }
    m = group_max<32>(m);
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int q = 0;
        if (m != 0.0f) {
            const float ratio = c[i] / m;                      // IEEE division
            q = (int)__builtin_rintf(__fmul_rn(ratio, 127.0f));
        }
        word |= ((uint32_t)(q & 0xFF)) << (8 * i);
    }
    if (base + 4 <= nb) {
        *reinterpret_cast<uint32_t*>(q8 + base) = word;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (base + i < nb) q8[base + i] = (int8_t)((word >> (8 * i)) & 0xFF);
    }
    if (lane == 0) scale[d] = m / 127.0f;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

size_t dq_workspace_bytes(int64_t nblocks) {
    size_t total = 0;
    int64_t cnt = cdiv(nblocks, kChunk);
    total += (size_t)cnt * sizeof(double);
    while (cnt > kChunk) {
        cnt = cdiv(cnt, kChunk);
        total += (size_t)cnt * sizeof(double);
    }
    return total;
}

hipError_t launch_double_quant(const float* absmax, int64_t nblocks, int8_t* q8, float* scale, float* mean,
                               void* workspace, hipStream_t s) {
    double* ws = reinterpret_cast<double*>(workspace);
    int64_t cnt = cdiv(nblocks, kChunk);
    hipLaunchKernelGGL(tree_partials<float>, dim3((unsigned)cnt), dim3(kThreads), 0, s, absmax, nblocks, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    double* cur = ws;
    while (cnt > kChunk) {
        const int64_t next = cdiv(cnt, kChunk);
        hipLaunchKernelGGL(tree_partials<double>, dim3((unsigned)next), dim3(kThreads), 0, s, cur, cnt, cur + cnt);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        cur += cnt;
        cnt = next;
    }
    const int64_t nd = cdiv(nblocks, kDqBlock);
    const int64_t grid = cdiv(nd, kDqBlocksPerWg);
    hipLaunchKernelGGL(dq_quantize, dim3((unsigned)grid), dim3(kThreads), 0, s, absmax, nblocks, cur, cnt, q8, scale,
                       mean);
    return hipGetLastError();
}

}  // namespace qk
