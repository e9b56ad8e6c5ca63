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
//     tree sum bit for bit.  The fp32 level reads 16 bytes per load from a
//     buffer range that ends at the array (the zero padding comes from the
//     range check).
//   dq_quantize: every workgroup first re-derives the mean from the final
//     partials (the same tree, at most 32 KB read from L2), then each of its 4
//     waves quantizes 4 blocks of 256 absmax (4 per lane), their loads issued
//     together.
#include <vector>

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dq_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int32_t)bytes, 0x00020000);
}

// First level over the fp32 absmax: thread t of the workgroup holds values [16 t, 16 t + 16)
// of the chunk, read with four 16-byte loads from a buffer whose range ends at the array's
// end (values past it read as zero: the tree's zero padding).  The 4-byte alignment of the
// array is enough for these loads.
__device__ __forceinline__ void partial_of_chunk(const float* __restrict__ in, int64_t count, int64_t chunk,
                                                 double* __restrict__ out, double* red) {
    const int64_t c0 = chunk * kChunk;
    const int64_t rem = count - c0;
    const __amdgpu_buffer_rsrc_t r = dq_rsrc(in + c0, 4 * (rem < kChunk ? rem : kChunk));
    double a[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
        const float4 v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        r, (uint32_t)(threadIdx.x * kPerThread * 4 + 16 * j), 0, 0));
        a[4 * j] = (double)v.x;
        a[4 * j + 1] = (double)v.y;
        a[4 * j + 2] = (double)v.z;
        a[4 * j + 3] = (double)v.w;
    }
    const double s = chunk_tree(a, red);
    if (threadIdx.x == 0) out[chunk] = s;
}

__global__ __launch_bounds__(kThreads) void tree_partials_f32(const float* __restrict__ in, int64_t count,
                                                              double* __restrict__ out) {
    __shared__ double red[kThreads / kWave];
    partial_of_chunk(in, count, blockIdx.x, out, red);
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
constexpr int kMaxDqGroup = 16;                  // arrays per grouped launch
constexpr int kDqPerWave = 4;                    // dq blocks a wave quantizes
constexpr int kDqBlocksPerWg = kThreads / kWave * kDqPerWave;

// Workgroup wg of the quantization of one array: the mean from its final partials, then
// the workgroup's kDqBlocksPerWg blocks of 256 (workgroup 0 also stores the mean).
__device__ __forceinline__ void dq_quantize_wg(const float* __restrict__ absmax, int64_t nb,
                                               const double* __restrict__ partials, int64_t npart,
                                               int8_t* __restrict__ q8, float* __restrict__ scale,
                                               float* __restrict__ mean_out, int64_t wg, double* red,
                                               float* mean_sh) {
    // mean from the final partials (npart <= 4096), same tree as the partial kernel; eight
    // 16-byte loads per thread, partials past npart read as zero
    {
        const __amdgpu_buffer_rsrc_t pr = dq_rsrc(partials, 8 * npart);
        double a[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread / 2; ++j) {
            const double2 v = __builtin_bit_cast(double2, __builtin_amdgcn_raw_buffer_load_b128(
                                                              pr, (uint32_t)(threadIdx.x * kPerThread * 8 + 16 * j), 0, 0));
            a[2 * j] = v.x;
            a[2 * j + 1] = v.y;
        }
        const double total = chunk_tree(a, red);
        if (threadIdx.x == 0) {
            const float mu = (float)(total / (double)nb);
            *mean_sh = mu;
            if (wg == 0) *mean_out = mu;
        }
        __syncthreads();
    }
    const float mu = *mean_sh;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nd = (nb + kDqBlock - 1) / kDqBlock;
    // this wave's kDqPerWave blocks: one 16-byte load per lane and block, all issued first
    // (the buffer ends at the array's end; values past it are masked below)
    const int64_t d0 = wg * kDqBlocksPerWg + (threadIdx.x / kWave) * kDqPerWave;
    if (d0 >= nd) return;
    const int64_t e0 = d0 * kDqBlock;
    const int64_t rem = nb - e0;
    const __amdgpu_buffer_rsrc_t ar = dq_rsrc(absmax + e0, 4 * (rem < kDqPerWave * kDqBlock ? rem : kDqPerWave * kDqBlock));
    float4 av[kDqPerWave];
#pragma unroll
    for (int k = 0; k < kDqPerWave; ++k)
        av[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ar, (uint32_t)(k * kDqBlock * 4 + 16 * lane), 0, 0));
#pragma unroll
    for (int k = 0; k < kDqPerWave; ++k) {
        const int64_t d = d0 + k;
        if (d >= nd) break;
        const int64_t base = d * kDqBlock + lane * 4;
        const float avk[4] = {av[k].x, av[k].y, av[k].z, av[k].w};
        float c[4];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = (base + i < nb) ? __fsub_rn(avk[i], mu) : 0.0f;
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
}

__global__ __launch_bounds__(kThreads) void dq_quantize(const float* __restrict__ absmax, int64_t nb,
                                                        const double* __restrict__ partials, int64_t npart,
                                                        int8_t* __restrict__ q8, float* __restrict__ scale,
                                                        float* __restrict__ mean_out) {
    __shared__ double red[kThreads / kWave];
    __shared__ float mean_sh;
    dq_quantize_wg(absmax, nb, partials, npart, q8, scale, mean_out, blockIdx.x, red, &mean_sh);
}

// Several arrays in one launch each: workgroup w of the launch belongs to the array t with
// first[t] <= w < first[t + 1] (a uniform search over at most kMaxDqGroup entries) and
// does that array's work item w - first[t], exactly as the single-array kernels do.
struct DqGroup {
    const float* absmax[kMaxDqGroup];
    double* part[kMaxDqGroup];       // the array's final (and only) level of partials
    int8_t* q8[kMaxDqGroup];
    float* scale[kMaxDqGroup];
    float* mean[kMaxDqGroup];
    int64_t nb[kMaxDqGroup];
    int32_t chunk0[kMaxDqGroup + 1]; // first workgroup of each array in the partials launch
    int32_t wg0[kMaxDqGroup + 1];    // first workgroup of each array in the quantization launch
    int32_t count;
};

__device__ __forceinline__ int dq_task_of(const int32_t* first, int32_t count, int32_t w) {
    int t = 0;
    while (t + 1 < count && w >= first[t + 1]) ++t;
    return t;
}

__global__ __launch_bounds__(kThreads) void tree_partials_f32_group(DqGroup g) {
    __shared__ double red[kThreads / kWave];
    const int32_t w = (int32_t)blockIdx.x;
    const int t = dq_task_of(g.chunk0, g.count, w);
    partial_of_chunk(g.absmax[t], g.nb[t], w - g.chunk0[t], g.part[t], red);
}

__global__ __launch_bounds__(kThreads) void dq_quantize_group(DqGroup g) {
    __shared__ double red[kThreads / kWave];
    __shared__ float mean_sh;
    const int32_t w = (int32_t)blockIdx.x;
    const int t = dq_task_of(g.wg0, g.count, w);
    const int64_t nb = g.nb[t];
    dq_quantize_wg(g.absmax[t], nb, g.part[t], (nb + kChunk - 1) / kChunk, g.q8[t], g.scale[t], g.mean[t],
                   w - g.wg0[t], red, &mean_sh);
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
    hipLaunchKernelGGL(tree_partials_f32, dim3((unsigned)cnt), dim3(kThreads), 0, s, absmax, nblocks, ws);
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

hipError_t launch_double_quant_group(const DqItem* items, int32_t count, void* workspace, hipStream_t s) {
    // each array's partials sit at its own offset of the workspace (the sizes are whole
    // doubles); an array whose partials take more than one level goes alone
    std::vector<size_t> offs((size_t)count);
    size_t off = 0;
    for (int32_t i = 0; i < count; ++i) {
        offs[(size_t)i] = off;
        off += dq_workspace_bytes(items[i].nblocks);
    }
    char* ws = reinterpret_cast<char*>(workspace);
    DqGroup g;
    auto flush = [&]() -> hipError_t {
        if (g.count == 0) return hipSuccess;
        hipLaunchKernelGGL(tree_partials_f32_group, dim3((unsigned)g.chunk0[g.count]), dim3(kThreads), 0, s, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(dq_quantize_group, dim3((unsigned)g.wg0[g.count]), dim3(kThreads), 0, s, g);
        e = hipGetLastError();
        g.count = 0;
        return e;
    };
    g.count = 0;
    g.chunk0[0] = 0;
    g.wg0[0] = 0;
    for (int32_t i = 0; i < count; ++i) {
        const DqItem& it = items[i];
        double* part = reinterpret_cast<double*>(ws + offs[(size_t)i]);
        const int64_t chunks = cdiv(it.nblocks, kChunk);
        if (chunks > kChunk) {
            const hipError_t e = launch_double_quant(it.absmax, it.nblocks, it.q8, it.scale, it.mean, part, s);
            if (e != hipSuccess) return e;
            continue;
        }
        const int64_t wgs = cdiv(cdiv(it.nblocks, kDqBlock), kDqBlocksPerWg);
        // launch sizes stay far below 2^31 workgroups: flush before they could not
        if (g.count == kMaxDqGroup || (int64_t)g.chunk0[g.count] + chunks > (1 << 30) ||
            (int64_t)g.wg0[g.count] + wgs > (1 << 30)) {
            const hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        const int t = g.count;
        g.absmax[t] = it.absmax;
        g.part[t] = part;
        g.q8[t] = it.q8;
        g.scale[t] = it.scale;
        g.mean[t] = it.mean;
        g.nb[t] = it.nblocks;
        g.chunk0[t + 1] = g.chunk0[t] + (int32_t)chunks;
        g.wg0[t + 1] = g.wg0[t] + (int32_t)wgs;
        g.count = t + 1;
    }
    return flush();
}

}  // namespace qk
