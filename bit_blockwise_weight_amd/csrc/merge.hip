// LoRA merge into the dequantized weight, for gfx950.
//
// "LLM 相關知識" (technicalnotes, tag qlora), section 8 LoRA 的合併 (Merge): a
// 4-bit weight cannot be added to a BF16 one, so it is dequantized to BF16, the
// LoRA product is added (W_new = W + A x B, here with the layer's scale s and W
// stored [N, K], so W + s (A B)^T), and W_new is BF16; it can then be quantized
// again for deployment (qk_quantize_blockwise).  Definition computed here:
//     D[n, k] = bf16(RN(level[code] * a'))         (exactly what qk_dequantize writes)
//     P[n, k] = sum_{j < r} B[j, n] * A[k, j]      fp32, j increasing, each product exact
//     W_new   = bf16(RN(D + RN(s * P)))
//
// Work layout: a workgroup owns 64 rows x 256 k; thread t owns rows 8 (t / 32) .. +8
// and k 8 (t % 32) .. +8, a tile of 8 x 8 sums.  The adapter is staged 16 ranks
// at a time: A transposed to [rank][k] and B as [rank][row], both fp32 in LDS;
// for each rank a thread reads 8 B values (one address per 32 threads: a
// broadcast) and 8 A values (consecutive for consecutive threads) and does 64
// FMAs.  fma(b, a, p) rounds once, like the fp32 add of the exact product.
#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

constexpr int kRows = 64;
constexpr int kCols = 256;
constexpr int kThreads = 256;
constexpr int kRankChunk = 16;
constexpr int kCopies = 32;

struct MergeArgs {
    DeqArgs w;
    int64_t N, K;
    const uint16_t* A;    // [K, r] bf16
    const uint16_t* B;    // [r, N] bf16
    int32_t r;
    float scale;
    uint16_t* out;        // [N, K] bf16
};

__device__ __forceinline__ float bf16f(uint16_t b) { return as_float((uint32_t)b << 16); }

template <bool kVec, bool kVecAB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void lora_merge_kernel(MergeArgs a) {
    __shared__ float At[kRankChunk][kCols];      // 16 KB
    __shared__ float Bs[kRankChunk][kRows];      // 4 KB
    __shared__ float lev[16 * kCopies];          // 2 KB
    const int tid = threadIdx.x;
    // copy t % 32 of levels t / 32 and t / 32 + 8 (both loaded before either is written)
    static_assert(kCopies == 32 && kThreads == 256, "the fill assumes 32 copies and 256 threads");
    {
        const float l0 = a.w.levels[tid / kCopies], l1 = a.w.levels[tid / kCopies + 8];
        lev[tid] = l0;
        lev[tid + kThreads] = l1;
    }

    const int64_t k0 = (int64_t)blockIdx.x * kCols;
    const int64_t n0 = (int64_t)blockIdx.y * kRows;
    const int rg = tid >> 5, kc = tid & 31;
    const int64_t N = a.N, K = a.K;
    const int r = a.r;

    float p[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) p[i][q] = 0.0f;

    // kVec: the epilogue's code words and block-scale inputs are loaded here, so their
    // latency passes under the adapter product (rows or k past the edge read a valid
    // address and are not stored)
    const int64_t kb = k0 + 8 * kc;
    uint32_t cwp[8];
    int32_t qp[8];
    float dp[8];
    if constexpr (kVec) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t n = n0 + 8 * rg + i;
            const int64_t e0 = (n < N ? n : N - 1) * K + (kb < K ? kb : K - 8);
            cwp[i] = *reinterpret_cast<const uint32_t*>(a.w.codes + e0 / 2);
            const int64_t blk = e0 >> a.w.blocksize_log2;
            if (a.w.nested) {
                qp[i] = a.w.q8[blk];
                dp[i] = a.w.dq_scale[blk / QK_DQ_BLOCK];
            } else {
                qp[i] = (int32_t)as_uint(a.w.absmax[blk]);
                dp[i] = 0.0f;
            }
        }
    }

    // the adapter product, 16 ranks per LDS chunk; the first chunk is peeled so the
    // block scales are formed from their early loads right after its staging, where
    // those loads have landed (the staging waits for loads issued after them)
    const float mean = a.w.nested ? *a.w.dq_mean : 0.0f;
    float scp[8];
    auto make_scales = [&] {
        if constexpr (kVec) {
#pragma unroll
            for (int i = 0; i < 8; ++i) scp[i] = a.w.nested ? __fadd_rn(__fmul_rn((float)qp[i], dp[i]), mean) : as_float((uint32_t)qp[i]);
        }
    };
    auto stage = [&](int j0, int nr) {
        // A: thread t stages row k0 + t of the tile (ranks j0 .. j0 + nr)
        const int64_t k = k0 + tid;
        if constexpr (kVecAB) {
            // r % 8 == 0 (nr is 8 or 16), A and B 16-byte aligned, N % 8 == 0
            const uint4* ap = reinterpret_cast<const uint4*>(a.A + (k < K ? k : K - 1) * r + j0);
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            const uint4 h0 = k < K ? ap[0] : z;
            const uint4 h1 = (k < K && nr == 16) ? ap[1] : z;
            const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
            for (int j = 0; j < kRankChunk; ++j) At[j][tid] = as_float((j & 1) ? (hw[j >> 1] & 0xFFFF0000u) : (hw[j >> 1] << 16));
            // B: 16 ranks x 64 rows as 8-element pieces, threads 0 .. 127
            if (tid < kRankChunk * kRows / 8) {
                const int j = tid >> 3, nn = 8 * (tid & 7);
                uint4 bv = z;
                if (j < nr && n0 + nn < N) bv = *reinterpret_cast<const uint4*>(a.B + (int64_t)(j0 + j) * N + n0 + nn);
                const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int t = 0; t < 8; ++t) Bs[j][nn + t] = as_float((t & 1) ? (bw[t >> 1] & 0xFFFF0000u) : (bw[t >> 1] << 16));
            }
        } else {
            for (int j = 0; j < kRankChunk; ++j)
                At[j][tid] = (k < K && j < nr) ? bf16f(a.A[k * r + j0 + j]) : 0.0f;
            // B: 16 ranks x 64 rows, 4 per thread
            for (int e = tid; e < kRankChunk * kRows; e += kThreads) {
                const int j = e / kRows, nn = e % kRows;
                Bs[j][nn] = (j < nr && n0 + nn < N) ? bf16f(a.B[(int64_t)(j0 + j) * N + n0 + nn]) : 0.0f;
            }
        }
    };
    auto ranks = [&](int nr) {
        for (int j = 0; j < nr; ++j) {
            const float4 b0 = *reinterpret_cast<const float4*>(&Bs[j][8 * rg]);
            const float4 b1 = *reinterpret_cast<const float4*>(&Bs[j][8 * rg + 4]);
            const float4 a0 = *reinterpret_cast<const float4*>(&At[j][8 * kc]);
            const float4 a1 = *reinterpret_cast<const float4*>(&At[j][8 * kc + 4]);
            const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q) p[i][q] = __builtin_fmaf(bv[i], av[q], p[i][q]);
        }
    };
    if (r > 0) {
        const int nr0 = r < kRankChunk ? r : kRankChunk;
        stage(0, nr0);
        __syncthreads();
        make_scales();
        ranks(nr0);
        for (int j0 = kRankChunk; j0 < r; j0 += kRankChunk) {
            const int nr = r - j0 < kRankChunk ? r - j0 : kRankChunk;
            __syncthreads();                               // the previous chunk has been read
            stage(j0, nr);
            __syncthreads();
            ranks(nr);
        }
    } else {
        __syncthreads();                                   // lev
        make_scales();
    }

    const int copy = tid & (kCopies - 1);
    auto scale_of = [&](int64_t blk) {
        return a.w.nested ? __fadd_rn(__fmul_rn((float)a.w.q8[blk], a.w.dq_scale[blk / QK_DQ_BLOCK]), mean)
                          : a.w.absmax[blk];
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t n = n0 + 8 * rg + i;
        if (n >= N || kb >= K) continue;
        const int64_t e0 = n * K + kb;
        float w[8];
        if constexpr (kVec) {
            // K % 8 == 0: the 8 elements are 4 aligned code bytes inside one block
            const uint32_t cw = cwp[i];
            const float sc = scp[i];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t code = (cw >> (8 * (q >> 1) + ((q & 1) ? 0 : 4))) & 0xFu;
                const float d = bf16_hi(pack_bf16x2(0.0f, __fmul_rn(lev[code * kCopies + copy], sc)));
                w[q] = __fadd_rn(d, __fmul_rn(a.scale, p[i][q]));
            }
            *reinterpret_cast<uint4*>(a.out + e0) = make_uint4(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                                                               pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7]));
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (kb + q >= K) break;
                const int64_t e = e0 + q;
                const uint32_t byte = a.w.codes[e >> 1];
                const uint32_t code = (e & 1) ? (byte & 0xFu) : (byte >> 4);
                const float d = bf16_hi(pack_bf16x2(0.0f, __fmul_rn(lev[code * kCopies + copy], scale_of(e >> a.w.blocksize_log2))));
                w[q] = __fadd_rn(d, __fmul_rn(a.scale, p[i][q]));
                a.out[e] = (uint16_t)(pack_bf16x2(w[q], 0.0f) & 0xFFFFu);
            }
        }
    }
}

}  // namespace

hipError_t launch_lora_merge(const MatArgs& w, const void* A, const void* B, int32_t r, float scale, void* out,
                             hipStream_t s) {
    MergeArgs a;
    a.w = w.w;
    a.N = w.N;
    a.K = w.K;
    a.A = reinterpret_cast<const uint16_t*>(A);
    a.B = reinterpret_cast<const uint16_t*>(B);
    a.r = r;
    a.scale = scale;
    a.out = reinterpret_cast<uint16_t*>(out);
    const int64_t gy = (w.N + kRows - 1) / kRows;
    if (gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((w.K + kCols - 1) / kCols), (unsigned)gy);
    const bool vec = (w.K % 8) == 0 && (reinterpret_cast<uintptr_t>(out) % 16) == 0;
    const bool vec_ab = (r % 8) == 0 && (w.N % 8) == 0 && (reinterpret_cast<uintptr_t>(A) % 16) == 0 &&
                        (reinterpret_cast<uintptr_t>(B) % 16) == 0;
    if (vec && vec_ab) hipLaunchKernelGGL((lora_merge_kernel<true, true>), grid, dim3(kThreads), 0, s, a);
    else if (vec) hipLaunchKernelGGL((lora_merge_kernel<true, false>), grid, dim3(kThreads), 0, s, a);
    else if (vec_ab) hipLaunchKernelGGL((lora_merge_kernel<false, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((lora_merge_kernel<false, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qk
