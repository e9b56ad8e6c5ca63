// Prefill / training GEMM of a frozen 4-bit base layer with an unmerged LoRA
// adapter, for gfx950:
//     Y = X · deq(W)^T + s · (X · A) · B
// "LLM 相關知識" (technicalnotes, tag qlora), sections 2-2 LoRA (W + ΔW with
// ΔW = A × B, A and B trainable BF16), 5 動態反量化 (the 4-bit base is restored to
// BF16 tile by tile just before the matmul) and 8 (without merging, base output
// and LoRA output are computed separately and added);
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 (QLoRA forward).
//
// Two kernels compute it, chosen per call:
//   * gemm_fast_kernel (the hot path: K a multiple of 64 and of the block size,
//     16-byte aligned X, Y and codes): 256 x 256 output tiles, one 8-wave workgroup
//     per CU, wave w owns weight rows 32w..32w+31 and all 256 token rows (8 tiles
//     of v_mfma_f32_32x32x16_bf16), so every weight is dequantized exactly once,
//     per lane and straight into MFMA B fragments (bf16 of RN(level * a'), the
//     value the dequantize kernel writes); X tiles enter two XOR-swizzled LDS
//     buffers by buffer loads with the LDS bit; the LoRA product s * X * A comes
//     from a K-split pre-pass (lora_xa_kernel) whose partials the epilogue sums in
//     split order and applies as bf16 hi + lo with two more MFMAs per tile.  The
//     pipeline and its measured limits are described next to the kernel below.
//     A grouped call (a layer's GEMMs) runs the pre-passes of its GEMMs in one
//     launch and their tiles in another, longest rows first; both kernels find
//     their GEMM in the launch's prefix table and run the single call's code.
//   * gemm_tile128_kernel (any other shape or alignment): 128 x 128 tiles, 4
//     waves as 2 x 2, each 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16; the
//     W tile is dequantized by the workgroup into LDS (flat indexing when blocks
//     straddle rows), X is copied to LDS (element by element in the generic
//     variant), T = X * A accumulates in the same K loop from the X tile in LDS
//     and (s T) * B is added after it as bf16 hi + lo.  LDS rows are padded to
//     144 bytes so the fragment reads of 8 consecutive rows fall in distinct banks.
// Both end with fp32 accumulators -> bf16 (RNE) -> Y.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kLdsStride = BK + 8;        // bf16 elements per LDS row (144 bytes)
constexpr int kMaxRank = 64;
constexpr int kMaxGemmGroup = 8;          // GEMMs of one grouped launch

struct GemmArgs {
    const uint16_t* X;   // [M, K]
    const uint16_t* A;   // [K, r] or null
    const uint16_t* B;   // [r, N] or null
    uint16_t* Y;         // [M, N]
    DeqArgs w;
    int64_t M, N, K;
    int32_t r;
    float lora_scale;
};

__device__ __forceinline__ float wscale(const DeqArgs& a, int64_t blk) {
    if (!a.nested) return a.absmax[blk];
    return __fadd_rn(__fmul_rn((float)a.q8[blk], a.dq_scale[blk / QK_DQ_BLOCK]), *a.dq_mean);
}

__device__ __forceinline__ uint32_t deq_pair(const float* lev, uint32_t byte, float sc) {
    // element 2t (high nibble) in the low half, element 2t+1 in the high half
    return pack_bf16x2(__fmul_rn(lev[byte >> 4], sc), __fmul_rn(lev[byte & 15u], sc));
}

// kVecGen (generic path, K < 2^22): X, codes and block scales of a step are fetched with
// 16-byte buffer loads from 4-byte aligned bases (rows past M and codes past the weight
// read zero through the range check; a row's elements past K are masked), not element by
// element; the dequantized values are the same.
template <bool kGeneric, bool kLora, bool kVecGen>
__global__ __launch_bounds__(kThreads) void gemm_tile128_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN * kLdsStride];
    __shared__ float lev[16];
    // LoRA: A^T tile [r_pad][BK] (bf16), and the s*T tile after the loop
    __shared__ __attribute__((aligned(16))) uint16_t as_[kLora ? kMaxRank * kLdsStride : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t M = a.M, N = a.N, K = a.K;
    if (tid < 16) lev[tid] = a.w.levels[tid];

    const int64_t nk = (K + BK - 1) / BK;
    const int rpad = kLora ? ((a.r + 15) / 16) * 16 : 0;

    // ---- per-thread global load assignment
    // X: 128 rows x 8 chunks of 16 B; thread takes chunks c = tid + 256 * v, v < 4
    // W: 128 rows x 2 halves; thread takes row tid / 2, half tid % 2
    const int wrow = tid >> 1, whalf = tid & 1;
    const int64_t wn_row = n0 + wrow;
    const bool wrow_ok = wn_row < N;

    uint4 xr[4];
    uint4 cr;
    float csc;
    uint16_t xg[kGeneric && !kVecGen ? 32 : 1];   // generic path: 32 X elements per thread
    uint32_t cg[kGeneric && !kVecGen ? 16 : 1];   // generic path: 16 packed code bytes (re-packed)
    float scg[kGeneric && !kVecGen ? 32 : 1];
    // vectorized generic path: the thread's 32 X elements as 16 words, its 32 codes as 4
    // words (first element in the high nibble), the block scales and where they change
    uint32_t xq[kVecGen ? 16 : 1];
    uint32_t cq[kVecGen ? 4 : 1];
    float vsc0 = 0.0f, vsc1 = 0.0f;
    int vsplit = 32, vlive = 32;
    // per-tile buffer resources over 4-byte aligned bases: X rows m0 .. m0 + BM and the
    // codes of weight rows n0 .. n0 + BN.  Each range is rounded up to whole dwords, so a
    // dword that holds the last element is read whole whichever way the hardware checks a
    // dword that straddles the end; the extra bytes share that dword's page and feed only
    // masked elements.
    __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(nullptr, (short)0, 0, 0x00020000);
    __amdgpu_buffer_rsrc_t crs = xrs;
    uint32_t x_mis = 0, c_mis = 0, c_phase0 = 0;
    if constexpr (kVecGen) {
        const uintptr_t xa = reinterpret_cast<uintptr_t>(a.X + m0 * K);
        x_mis = (uint32_t)(xa & 3u);
        const int64_t xrows = M - m0 < BM ? M - m0 : BM;
        xrs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(xa - x_mis), (short)0,
                                               (int32_t)((xrows * K * 2 + x_mis + 3) & ~3LL), 0x00020000);
        const int64_t cfirst = n0 * K;                       // flat element of the tile's first weight
        const uintptr_t ca = reinterpret_cast<uintptr_t>(a.w.codes + (cfirst >> 1));
        c_mis = (uint32_t)(ca & 3u);
        c_phase0 = (uint32_t)(cfirst & 1);
        const int64_t wrows = N - n0 < BN ? N - n0 : BN;
        const int64_t cend = (cfirst + wrows * K + 1) >> 1;  // bytes of the tile's weights end here
        crs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ca - c_mis), (short)0,
                                               (int32_t)((cend - (cfirst >> 1) + c_mis + 3) & ~3LL), 0x00020000);
    }
    constexpr int kAPer = kLora ? kMaxRank * BK / kThreads : 1;   // 16
    uint16_t ag[kAPer];               // LoRA A^T elements owned by this thread
    // vectorized generic path with r % 8 == 0: the step's A rows k0 .. k0 + 64 are one
    // contiguous run of 64 r elements; piece p = tid + 256 v holds its elements 8 p .. 8 p + 8,
    // which lie in one row kk = 8 p / r, ranks 8 p % r + [0, 8)
    constexpr int kAPieces = kLora ? kMaxRank * BK / 8 / kThreads : 1;   // 2
    uint32_t aq[kAPieces][4];
    int64_t vk0 = 0;                  // the k0 of the pieces in aq
    const bool a_vec = kVecGen && kLora && (a.r % 8) == 0;
    __amdgpu_buffer_rsrc_t ars = xrs;
    uint32_t a_mis = 0;
    if constexpr (kVecGen && kLora) {
        if (a_vec) {
            const uintptr_t aa = reinterpret_cast<uintptr_t>(a.A);
            a_mis = (uint32_t)(aa & 3u);
            ars = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(aa - a_mis), (short)0,
                                                   (int32_t)((K * a.r * 2 + a_mis + 3) & ~3LL), 0x00020000);
        }
    }

    auto load_step = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
        if constexpr (!kGeneric) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int c = tid + kThreads * v;
                const int row = c >> 3, ch = c & 7;
                const int64_t gm = m0 + row;
                xr[v] = gm < M ? *reinterpret_cast<const uint4*>(a.X + gm * K + k0 + ch * 8) : make_uint4(0, 0, 0, 0);
            }
            const int64_t e0 = wn_row * K + k0 + whalf * 32;
            if (wrow_ok) {
                cr = *reinterpret_cast<const uint4*>(a.w.codes + e0 / 2);
                csc = wscale(a.w, e0 >> a.w.blocksize_log2);
            } else {
                cr = make_uint4(0, 0, 0, 0);
                csc = 0.0f;
            }
        } else if constexpr (kVecGen) {
            // X: row tid / 2 of the tile, elements k0 + 32 h + [0, 32): 17 words from the
            // 4-byte aligned byte offset, shifted by one half word when the row starts there
            {
                const int row = tid >> 1, h = tid & 1;
                const uint32_t xb = x_mis + 2u * (uint32_t)(row * K + k0 + 32 * h);
                const uint32_t xb4 = xb & ~3u;
                uint32_t w[17];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, xb4 + 16u * q, 0, 0));
                    w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
                }
                w[16] = __builtin_amdgcn_raw_buffer_load_b32(xrs, xb4 + 64u, 0, 0);
                const uint32_t sh = xb & 2u;
#pragma unroll
                for (int j = 0; j < 16; ++j) xq[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], sh);
                // elements past the row's end (the last step of a K that is not a multiple of 64)
                const int64_t kb = k0 + 32 * h;
                if (kb + 32 > K) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const uint32_t lo = kb + 2 * j < K ? 0x0000FFFFu : 0u;
                        const uint32_t hi = kb + 2 * j + 1 < K ? 0xFFFF0000u : 0u;
                        xq[j] &= lo | hi;
                    }
                }
            }
            // W: weight row n0 + tid / 2, elements k0 + 32 whalf + [0, 32) (flat er from the
            // tile's first weight): 20 bytes from the aligned byte offset, the 16 or 17 bytes of
            // the run realigned, the nibble stream moved by one when the run starts odd
            {
                const uint32_t er = (uint32_t)(wrow * K + k0 + 32 * whalf);
                const uint32_t ep = c_phase0 + er;                  // from the tile's first byte
                const uint32_t cb = c_mis + (ep >> 1);
                const uint32_t cb4 = cb & ~3u;
                const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cb4, 0, 0));
                const uint32_t w4 = __builtin_amdgcn_raw_buffer_load_b32(crs, cb4 + 16u, 0, 0);
                const uint32_t w[5] = {v[0], v[1], v[2], v[3], w4};
                const uint32_t csh = cb & 3u;
                uint32_t o[5];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], csh);
                o[4] = w[4] >> (8u * csh);
                if (ep & 1u) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        cq[j] = ((o[j] << 4) & 0xF0F0F0F0u) | ((__builtin_amdgcn_alignbyte(o[j + 1], o[j], 1) >> 4) & 0x0F0F0F0Fu);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) cq[j] = o[j];
                }
                // block scales: the run's elements fall in the block of its first element and
                // perhaps the next; elements past the row's end (and rows past N) get scale 0
                const int64_t e0 = wn_row * K + k0 + 32 * whalf;
                const int64_t kb = k0 + 32 * whalf;
                vlive = !wrow_ok ? 0 : (kb + 32 <= K ? 32 : (kb < K ? (int)(K - kb) : 0));
                if (vlive > 0) {
                    const int64_t blk0 = e0 >> a.w.blocksize_log2;
                    const int64_t into = e0 & (a.w.blocksize - 1);
                    vsplit = a.w.blocksize - into < 32 ? (int)(a.w.blocksize - into) : 32;
                    vsc0 = wscale(a.w, blk0);
                    vsc1 = vsplit < vlive ? wscale(a.w, blk0 + 1) : vsc0;
                }
            }
        } else {
            // X: thread handles row tid/2, 32 elements starting at (tid%2)*32
            const int row = tid >> 1, h = tid & 1;
            const int64_t gm = m0 + row;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int64_t k = k0 + h * 32 + i;
                xg[i] = (gm < M && k < K) ? a.X[gm * K + k] : (uint16_t)0;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) cg[i] = 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int64_t k = k0 + whalf * 32 + i;
                uint32_t code = 0;
                float sc = 0.0f;
                if (wrow_ok && k < K) {
                    const int64_t e = wn_row * K + k;
                    const uint32_t byte = a.w.codes[e >> 1];
                    code = (e & 1) ? (byte & 0xFu) : (byte >> 4);
                    sc = wscale(a.w, e >> a.w.blocksize_log2);
                }
                cg[i >> 1] |= code << ((i & 1) ? 0 : 4);
                scg[i] = sc;
            }
        }
        if constexpr (kLora && kVecGen) {
            if (a_vec) {
                vk0 = k0;
#pragma unroll
                for (int v = 0; v < kAPieces; ++v) {
                    const uint32_t p = (uint32_t)(tid + kThreads * v);
                    const uint32_t ab = a_mis + 2u * (uint32_t)(k0 * a.r + 8 * p);
                    const uint32_t ab4 = ab & ~3u;
                    const u32x4_t w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ars, ab4, 0, 0));
                    const uint32_t w4 = __builtin_amdgcn_raw_buffer_load_b32(ars, ab4 + 16u, 0, 0);
                    const uint32_t ww[5] = {w[0], w[1], w[2], w[3], w4};
#pragma unroll
                    for (int q = 0; q < 4; ++q) aq[v][q] = __builtin_amdgcn_alignbyte(ww[q + 1], ww[q], ab & 2u);
                }
                return;
            }
        }
        if constexpr (kLora) {
            // A^T tile: [rpad][BK]; thread covers elements e = tid + 256 * v of rpad*BK
#pragma unroll
            for (int v = 0; v < kAPer; ++v) {
                const int e = tid + kThreads * v;
                const int j = e / BK, kk = e % BK;
                const int64_t k = k0 + kk;
                ag[v] = (j < a.r && e < rpad * BK && k < K) ? a.A[k * a.r + j] : (uint16_t)0;
            }
        }
    };

    auto store_step = [&](int buf) {
        if constexpr (!kGeneric) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int c = tid + kThreads * v;
                const int row = c >> 3, ch = c & 7;
                *reinterpret_cast<uint4*>(&xs[buf][row * kLdsStride + ch * 8]) = xr[v];
            }
            const uint32_t cw[4] = {cr.x, cr.y, cr.z, cr.w};
            uint32_t o[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int b = 0; b < 4; ++b) o[4 * q + b] = deq_pair(lev, (cw[q] >> (8 * b)) & 0xFFu, csc);
            }
            uint4* dst = reinterpret_cast<uint4*>(&ws[buf][wrow * kLdsStride + whalf * 32]);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else if constexpr (kVecGen) {
            const int row = tid >> 1, h = tid & 1;
            uint4* xd = reinterpret_cast<uint4*>(&xs[buf][row * kLdsStride + h * 32]);
#pragma unroll
            for (int q = 0; q < 4; ++q) xd[q] = make_uint4(xq[4 * q], xq[4 * q + 1], xq[4 * q + 2], xq[4 * q + 3]);
            uint32_t o[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const uint32_t byte = (cq[m >> 2] >> (8 * (m & 3))) & 0xFFu;
                const int i0 = 2 * m, i1 = 2 * m + 1;
                const float s0 = i0 < vlive ? (i0 < vsplit ? vsc0 : vsc1) : 0.0f;
                const float s1 = i1 < vlive ? (i1 < vsplit ? vsc0 : vsc1) : 0.0f;
                o[m] = pack_bf16x2(__fmul_rn(lev[byte >> 4], s0), __fmul_rn(lev[byte & 15u], s1));
            }
            uint4* dst = reinterpret_cast<uint4*>(&ws[buf][wrow * kLdsStride + whalf * 32]);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
            const int row = tid >> 1, h = tid & 1;
#pragma unroll
            for (int i = 0; i < 32; ++i) xs[buf][row * kLdsStride + h * 32 + i] = xg[i];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const uint32_t code = (cg[i >> 1] >> ((i & 1) ? 0 : 4)) & 0xFu;
                ws[buf][wrow * kLdsStride + whalf * 32 + i] =
                    (uint16_t)(pack_bf16x2(__fmul_rn(lev[code], scg[i]), 0.0f) & 0xFFFFu);
            }
        }
        if constexpr (kLora && kVecGen) {
            if (a_vec) {
                // the step's k0 is the one loaded for this buffer: rows past K are zero
#pragma unroll
                for (int v = 0; v < kAPieces; ++v) {
                    const int p = tid + kThreads * v;
                    if (p >= 8 * a.r) continue;
                    const int kk = (8 * p) / a.r, j0 = (8 * p) % a.r;
                    const bool live = vk0 + kk < K;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        as_[(j0 + i) * kLdsStride + kk] = live ? (uint16_t)(aq[v][i >> 1] >> ((i & 1) ? 16 : 0)) : (uint16_t)0;
                }
                return;
            }
        }
        if constexpr (kLora) {
#pragma unroll
            for (int v = 0; v < kAPer; ++v) {
                const int e = tid + kThreads * v;
                if (e < rpad * BK) as_[(e / BK) * kLdsStride + (e % BK)] = ag[v];
            }
        }
    };

    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // LoRA T accumulators: this wave owns T rows [32*wave, 32*wave + 32) as 2 x (rpad/16) 16x16 tiles
    floatx4_t tacc[2][kMaxRank / 16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kMaxRank / 16; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) tacc[i][j][r] = 0.0f;

    if constexpr (kLora && kVecGen) {
        // ranks r .. rpad of the A^T tile stay zero: the vectorized stores never write them
        if (a_vec) {
            for (int e = tid; e < (rpad - a.r) * BK; e += kThreads)
                as_[(a.r + e / BK) * kLdsStride + (e % BK)] = (uint16_t)0;
        }
    }
    __syncthreads();   // lev ready
    load_step(0);
    store_step(0);
    __syncthreads();

    const int fi = lane & 31;         // fragment row / column within a 32 tile
    const int fg = lane >> 5;         // k half (8 elements) within a 16-k MFMA step
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk) load_step(kt + 1);
        const uint16_t* xb = xs[buf];
        const uint16_t* wb = ws[buf];
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + fi;
                af[i] = *reinterpret_cast<const bf16x8_t*>(&xb[row * kLdsStride + kk + 8 * fg]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wn * 64 + j * 32 + fi;
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&wb[col * kLdsStride + kk + 8 * fg]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if constexpr (kLora) {
            // T[32*wave + 16i + (l%16)][16j + ..] += X[..][k] A[k][..], 16x16x32 tiles
            const int l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
            for (int kk = 0; kk < BK; kk += 32) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wave * 32 + i * 16 + l16;
                    const bf16x8_t xa = *reinterpret_cast<const bf16x8_t*>(&xb[row * kLdsStride + kk + 8 * q4]);
#pragma unroll
                    for (int j = 0; j < kMaxRank / 16; ++j) {
                        if (16 * j >= rpad) break;
                        const bf16x8_t ab =
                            *reinterpret_cast<const bf16x8_t*>(&as_[(16 * j + l16) * kLdsStride + kk + 8 * q4]);
                        tacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ab, tacc[i][j], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
        if (kt + 1 < nk) {
            store_step(buf ^ 1);
            __syncthreads();
        }
    }

    if constexpr (kLora) {
        // s*T -> LDS as bf16 hi / lo: tl[row][j] (row < 128, j < rpad), stored in xs[0] / xs[1]
        uint16_t* thi = xs[0];
        uint16_t* tlo = xs[1];
        const int l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int j = 0; j < kMaxRank / 16; ++j) {
                if (16 * j >= rpad) break;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // 16x16 output: lane holds C[4*(l/16) + r][l%16]
                    const int row = wave * 32 + i * 16 + 4 * q4 + r;
                    const int col = 16 * j + l16;
                    const float v = tacc[i][j][r] * a.lora_scale;
                    const uint32_t hb = pack_bf16x2(v, 0.0f) & 0xFFFFu;
                    const float h = as_float(hb << 16);
                    const uint32_t lb = pack_bf16x2(v - h, 0.0f) & 0xFFFFu;
                    thi[row * kLdsStride + col] = (uint16_t)hb;
                    tlo[row * kLdsStride + col] = (uint16_t)lb;
                }
            }
        }
        // B^T tile [BN][rpad] into ws[0]
        for (int e = tid; e < BN * rpad; e += kThreads) {
            const int col = e / rpad, j = e % rpad;
            const int64_t gn = n0 + col;
            ws[0][col * kLdsStride + j] = (j < a.r && gn < N) ? a.B[(int64_t)j * N + gn] : (uint16_t)0;
        }
        __syncthreads();
        for (int kk = 0; kk < rpad; kk += 16) {
            bf16x8_t ah[2], al[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + fi;
                ah[i] = *reinterpret_cast<const bf16x8_t*>(&thi[row * kLdsStride + kk + 8 * fg]);
                al[i] = *reinterpret_cast<const bf16x8_t*>(&tlo[row * kLdsStride + kk + 8 * fg]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wn * 64 + j * 32 + fi;
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&ws[0][col * kLdsStride + kk + 8 * fg]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bfr[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bfr[j], acc[i][j], 0, 0, 0);
                }
        }
    }

    // epilogue: lane holds C[8b + 4*(l/32) + q][l%32] in register 4b + q
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t gn = n0 + wn * 64 + j * 32 + fi;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r / 4) + 4 * fg + (r % 4);
                const int64_t gm = m0 + wm * 64 + i * 32 + row;
                if (gm < M && gn < N) a.Y[gm * N + gn] = (uint16_t)(pack_bf16x2(acc[i][j][r], 0.0f) & 0xFFFFu);
            }
        }
    }
}

template <bool kGeneric, bool kVecGen>
hipError_t launch_typed(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    if (a.A)
        hipLaunchKernelGGL((gemm_tile128_kernel<kGeneric, true, kVecGen>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_tile128_kernel<kGeneric, false, kVecGen>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fast path: 256 x 256 output tile, K step 64, 8 waves (two per SIMD, so one
// wave's dequantization runs while the other's MFMAs do).  Wave w owns weight
// rows [32w, 32w + 32) of the tile (one 32-column MFMA tile) and all 256 token
// rows (eight 32-row MFMA tiles), so each weight of the tile is dequantized by
// exactly one lane of one wave, straight into MFMA B-fragment registers:
//   lane l = (j = l % 32, g = l / 32) holds the 16 code bytes of weights
//   [64s + 32g, 64s + 32g + 32) of its row (one absmax block); a byte is looked
//   up in an LDS table of fp32 level pairs (32 interleaved copies, address built
//   by one v_perm), multiplied by the block's a' and rounded to bf16 — the same
//   bf16(RN(level * a')) that qk_dequantize writes.  Quarter q of the step (8
//   weights) is the B operand of the q-th 16-deep MFMA; the A operand is
//   X[row][64s + 32g + 8q .. +8] from LDS, the same k order.
// Pipeline:
//   * X tiles go into two LDS buffers by buffer loads with the LDS bit; the codes
//     are loaded into registers two steps ahead;
//   * in a quarter, each MFMA is followed by the read of its row tile's A fragment
//     for the next quarter; halfway through, the next quarter's B fragment is
//     scaled from table reads issued a quarter earlier, and the table reads for the
//     quarter after it are issued;
//   * one barrier per step, after its third quarter: by then every wave has read
//     the step's X buffer (it can take X of step s + 2) and X of step s + 1 has
//     landed (the fourth quarter reads the next step's first A fragments).
// X rows are 128 bytes in LDS with the 16-byte chunks XOR-swizzled by the row
// (chunk c of row r sits in slot c ^ ((r >> 1) & 7)), so the fragment reads of
// 16 consecutive rows hit 16 different bank groups (no LDS bank conflicts).
// Measured limit: per step a CU issues 256 16-byte and 128 8-byte LDS reads (every
// wave reads the whole X tile) plus the 32 KB X copy, about 1800 LDS cycles next to
// the 2048 cycles of its SIMDs' 64 MFMAs each, and the steady state runs at about
// two thirds of the MFMA rate the clock allows under this load (about 1.6 GHz).
// ---------------------------------------------------------------------------
namespace v4 {

constexpr int TM = 256;
constexpr int TN = 256;
constexpr int TK = 64;
constexpr int kCopies = 32;
constexpr int kSplits = 8;                // K splits of the LoRA X*A pre-pass
constexpr int kXcds = 8;                  // MI355X: 8 XCDs, workgroups dealt round robin
constexpr int kGroupM = 4;                // tile rows per group in the tile order

typedef __attribute__((address_space(3))) void* lptr_t;

// The GEMMs of one launch (a single call is a group of one): task t owns the
// workgroups [tile0[t], tile0[t + 1]) and reads its LoRA partials at T[t].
struct GemmGroup {
    GemmArgs t[kMaxGemmGroup];
    const float* T[kMaxGemmGroup];
    int32_t tile0[kMaxGemmGroup + 1];
    int32_t count;
};

__device__ __forceinline__ uint32_t xoff(int row, int chunk) {   // byte offset in an X tile
    return (uint32_t)(row * 8 + (chunk ^ ((row >> 1) & 7))) * 16u;
}

template <int R16, bool kNested>
__global__ __launch_bounds__(512, 1) void gemm_fast_kernel(GemmGroup gg) {
    constexpr int kThr = 512;                          // 8 waves, two per SIMD
    constexpr int kRp = 16 * R16;
    constexpr int kTs = 16 + 8;                        // row pitch of a staged 16-rank chunk of s X A
    // The chunks of s X A (16 ranks each) are staged after the K loop: staging the
    // first one in the prologue keeps its registers live across the loop, and the
    // rank-16 kernel then spills around it (measured 1-3% slower).
    constexpr int kCodeLoads = kNested ? 3 : 2;     // global loads issued by load_codes
    // Separate LDS objects: the compiler then knows that reads of one X buffer, of the
    // table or of the LoRA chunk never alias the loads into the other X buffer, and does
    // not wait for those loads before every LDS read.  The table has the largest
    // alignment, so it sits at LDS address 0 and its byte addresses are the v_perm
    // results themselves.
    __shared__ __attribute__((aligned(1024))) uint4 xsA[TM * 8];          // X tile buffer 0, 32 KB
    __shared__ __attribute__((aligned(1024))) uint4 xsB[TM * 8];          // X tile buffer 1, 32 KB
    __shared__ __attribute__((aligned(65536))) uint2 tab[256 * kCopies];  // fp32 level pairs, 64 KB
    __shared__ __attribute__((aligned(16))) uint16_t tst[2 * TM * kTs];   // s X A chunk, bf16 hi | lo, 24 KB

    // this workgroup's task (uniform: a scalar search of the launch's prefix table)
    int task = 0;
    while (task + 1 < gg.count && (int32_t)blockIdx.x >= gg.tile0[task + 1]) ++task;
    const GemmArgs& a = gg.t[task];
    const float* __restrict__ T = gg.T[task];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;
    const int g = lane >> 5;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t nk = K / TK, nk1 = nk - 1;
    const int r = a.r;
    int64_t m0, n0;
    {
        const uint32_t tiles_n = (uint32_t)((N + TN - 1) / TN), tiles_m = (uint32_t)((M + TM - 1) / TM);
        const uint32_t nt = tiles_n * tiles_m;
        const uint32_t bid = blockIdx.x - (uint32_t)gg.tile0[task];
        const uint32_t lid = (nt % kXcds == 0) ? (bid % kXcds) * (nt / kXcds) + bid / kXcds : bid;
        const uint32_t per_group = kGroupM * tiles_n;
        const uint32_t first_m = (lid / per_group) * kGroupM;
        const uint32_t gm = tiles_m - first_m < (uint32_t)kGroupM ? tiles_m - first_m : (uint32_t)kGroupM;
        const uint32_t in_group = lid % per_group;
        m0 = (int64_t)(first_m + in_group % gm) * TM;
        n0 = (int64_t)(in_group / gm) * TN;
    }
    {
        // entry of byte b = 16 hi + lo: (level[hi], level[lo]).  Thread t writes copy t % 32
        // of the bytes with lo = t / 32, for every hi: the lo level is loaded once and the
        // hi levels are uniform (scalar loads), so the fill costs one memory round trip
        static_assert(kCopies == 32, "the fill assumes 32 copies and 512 threads");
        const int c = tid & (kCopies - 1), lo = tid / kCopies;
        const uint32_t l0 = as_uint(a.w.levels[lo]);
#pragma unroll
        for (int hi = 0; hi < 16; ++hi) tab[(16 * hi + lo) * kCopies + c] = make_uint2(as_uint(a.w.levels[hi]), l0);
    }

    // this wave's 32 weight rows (one MFMA column tile)
    const int64_t wrow = n0 + 32 * wave + j;
    const bool wok = wrow < N;
    const int64_t wrow_c = wok ? wrow : N - 1;
    const uint32_t lane_sel = (uint32_t)(lane & (kCopies - 1)) * 8u;
    const char* tabb = reinterpret_cast<const char*>(tab);
    const float mean = kNested ? *a.w.dq_mean : 0.0f;

    uint16_t* thi = tst;
    uint16_t* tlo = tst + TM * kTs;
    auto load_lora_b = [&](int kk) {
        uint32_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int jj = kk + 8 * g + t;
            e[t] = (uint32_t)a.B[(int64_t)(jj < r ? jj : r - 1) * N + wrow_c];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (kk + 8 * g + t < r) ? e[t] : 0u;
        return __builtin_bit_cast(bf16x8_t, make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                                       e[4] | (e[5] << 16), e[6] | (e[7] << 16)));
    };
    auto stage_t = [&](int kk) {
        if (tid < TM) {
            const int64_t gm = m0 + tid < M ? m0 + tid : M - 1;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                float4 sum = *reinterpret_cast<const float4*>(T + gm * kRp + kk + 4 * c4);
#pragma unroll
                for (int sp = 1; sp < kSplits; ++sp) {
                    const float4 t = *reinterpret_cast<const float4*>(T + (sp * M + gm) * kRp + kk + 4 * c4);
                    sum.x += t.x; sum.y += t.y; sum.z += t.z; sum.w += t.w;
                }
                const uint32_t h01 = pack_bf16x2(sum.x, sum.y), h23 = pack_bf16x2(sum.z, sum.w);
                const uint32_t l01 = pack_bf16x2(sum.x - as_float(h01 << 16), sum.y - as_float(h01 & 0xFFFF0000u));
                const uint32_t l23 = pack_bf16x2(sum.z - as_float(h23 << 16), sum.w - as_float(h23 & 0xFFFF0000u));
                *reinterpret_cast<uint2*>(&thi[tid * kTs + 4 * c4]) = make_uint2(h01, h23);
                *reinterpret_cast<uint2*>(&tlo[tid * kTs + 4 * c4]) = make_uint2(l01, l23);
            }
        }
    };

    // X tiles: buffer loads with the LDS bit, 4 pieces of 16 bytes per lane and step.
    // Unlike the global (FLAT-encoded) form, these do not make the compiler drain every
    // LDS-read wait to zero while they are in flight.  The resource covers the tile's
    // rows; offsets are bytes from the tile's first row (rows past M are clamped to the
    // last row: they only feed output rows that are never stored).
    // Piece v of a lane is row 64 v + 8 wave + lane / 8 of the tile, so the pieces are a
    // uniform 64 rows apart.  The row part of the offset (row and piece) is in the vector
    // offset, which the range check covers, and only the step's k offset is in the scalar
    // offset, which it does not cover: a row past M has a vector offset at or beyond the
    // resource's size, so its load returns zero and touches no memory, and a row inside
    // the tile stays inside its own row for every k.
    const uint16_t* xtile = a.X + m0 * K;
    const int64_t xrows = M - m0 < TM ? M - m0 : TM;
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xtile), (short)0, (int)(xrows * K * 2), 0x00020000);
    uint32_t xsrc0;
    {
        const int p = wave * 64 + lane;                    // LDS 16-byte slot written by this lane (piece 0)
        const int row = p >> 3, slot = p & 7;
        const int chunk = slot ^ ((row >> 1) & 7);         // the same for every piece: rows differ by 64
        xsrc0 = (uint32_t)((row * K + chunk * 8) * 2);
    }
    const int32_t xstride = (int32_t)(64 * K * 2);
    auto load_x = [&](int64_t s, auto buf) {
        const int32_t kbytes = (int32_t)((s < nk1 ? s : nk1) * TK * 2);
        char* base = reinterpret_cast<char*>(decltype(buf)::value ? xsB : xsA);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            lptr_t dst = (lptr_t)((__attribute__((address_space(3))) char*)base + (v * 8 + wave) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, dst, 16, (int32_t)(xsrc0 + (uint32_t)(v * xstride)), kbytes, 0, 0);
        }
    };

    struct Codes {
        uint4 c;
        int32_t q;
        float d;
    };
    auto load_codes = [&](int64_t s, Codes& cs) {
        const int64_t k0 = (s < nk1 ? s : nk1) * TK;
        const int64_t e0 = wrow_c * K + k0 + 32 * g;
        const int64_t blk = e0 >> a.w.blocksize_log2;
        cs.c = *reinterpret_cast<const uint4*>(a.w.codes + e0 / 2);
        if constexpr (kNested) {
            cs.q = (int32_t)a.w.q8[blk];
            cs.d = a.w.dq_scale[blk / QK_DQ_BLOCK];
        } else {
            cs.q = (int32_t)as_uint(a.w.absmax[blk]);
            cs.d = 1.0f;
        }
    };
    auto scale_of = [&](const Codes& cs) {
        float sc;
        if constexpr (kNested) sc = __fadd_rn(__fmul_rn((float)cs.q, cs.d), mean);
        else sc = as_float((uint32_t)cs.q);
        return sc;
    };
    auto lookup_q = [&](const Codes& cs, int q, uint2 (&lv)[4]) {
        const uint32_t cw = q == 0 ? cs.c.x : q == 1 ? cs.c.y : q == 2 ? cs.c.z : cs.c.w;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint32_t addr = __builtin_amdgcn_perm(cw, lane_sel, 0x0C0C0400u | ((uint32_t)(4 + bb) << 8));
            lv[bb] = *reinterpret_cast<const uint2*>(tabb + addr);
        }
    };
    auto finish_q = [&](float sc, const uint2 (&lv)[4]) {
        uint32_t d[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) d[bb] = pack_bf16x2(__fmul_rn(as_float(lv[bb].x), sc), __fmul_rn(as_float(lv[bb].y), sc));
        return __builtin_bit_cast(bf16x8_t, make_uint4(d[0], d[1], d[2], d[3]));
    };

    floatx16_t acc[8];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rt][e] = 0.0f;

    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    Codes c0, c1, c2;              // codes of steps s .. s + 2
    load_codes(0, c0);
    load_codes(1, c1);
    load_x(0, Buf0{});
    load_x(1, Buf1{});
    // table and X(0) in LDS; X(1) (the last 4 loads) stays in flight
    __builtin_amdgcn_s_waitcnt(4 | 0x70);   // vmcnt(4) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // A fragments of the current quarter; each is replaced by the next quarter's right
    // after its MFMA is issued
    bf16x8_t af[8];
    uint2 lv[4];                   // table reads of the B fragment two quarters ahead
    bf16x8_t bq;
    {
        const char* xbb = reinterpret_cast<const char*>(xsA);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) af[rt] = *reinterpret_cast<const bf16x8_t*>(xbb + xoff(32 * rt + j, 4 * g));
        lookup_q(c0, 0, lv);
        bq = finish_q(scale_of(c0), lv);
        lookup_q(c0, 1, lv);
    }

    // One quarter, in this order (the scheduling barriers keep it): for each row tile its
    // MFMA and the read of its A fragment for the next quarter; after the fourth, the
    // scaling of the next quarter's B fragment (from table reads issued half a quarter
    // earlier) and the table reads for the quarter after it.  LDS reads return in order;
    // with this order every MFMA's wait leaves the 11 reads issued after its A fragment
    // outstanding, and the scaling waits only for table reads 4 MFMAs old.
    auto quarter = [&](const uint4* xa, int qa, float sc_cur, const Codes& cs_nn, int qnn) {
        const char* xbb = reinterpret_cast<const char*>(xa);
        bf16x8_t bn;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rt], bq, acc[rt], 0, 0, 0);
            af[rt] = *reinterpret_cast<const bf16x8_t*>(xbb + xoff(32 * rt + j, 4 * g + qa));
            if (rt == 3) {
                bn = finish_q(sc_cur, lv);
                lookup_q(cs_nn, qnn, lv);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        bq = bn;
    };
    // One K step: ca = codes of step s, cb = codes of step s + 1, cn receives the codes
    // of step s + 2; X of step s is in buffer s % 2, X of step s + 1 is on its way into
    // the other buffer.
    auto step = [&](int64_t s, auto buf, const Codes& ca, const Codes& cb, Codes& cn) {
        constexpr bool kB = decltype(buf)::value;
        const uint4* xcur = kB ? xsB : xsA;
        const uint4* xnxt = kB ? xsA : xsB;
        load_codes(s + 2, cn);
        const float sa = scale_of(ca);
        __builtin_amdgcn_sched_barrier(0);
        quarter(xcur, 1, sa, ca, 2);
        quarter(xcur, 2, sa, ca, 3);
        quarter(xcur, 3, sa, cb, 0);
        // X(s + 1) has landed once at most the code loads of step s + 2 are outstanding.
        // A plain s_barrier: __syncthreads() would add a release fence, which waits for
        // every outstanding global load.
        __builtin_amdgcn_s_waitcnt(kCodeLoads | 0x70);   // vmcnt(kCodeLoads) expcnt(7) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kB) load_x(s + 2, Buf1{});
        else load_x(s + 2, Buf0{});
        const float sb = scale_of(cb);
        __builtin_amdgcn_sched_barrier(0);
        quarter(xnxt, 0, sb, cb, 1);
    };
    // whole groups of 6 steps (3 code sets x 2 X buffers) without conditions inside (a
    // condition between steps merges the compiler's wait-count state across paths and
    // makes its waits conservative), then the 0-5 remaining steps
    const int64_t nk6 = nk - nk % 6;
    int64_t s = 0;
    for (; s < nk6; s += 6) {
        step(s, Buf0{}, c0, c1, c2);
        step(s + 1, Buf1{}, c1, c2, c0);
        step(s + 2, Buf0{}, c2, c0, c1);
        step(s + 3, Buf1{}, c0, c1, c2);
        step(s + 4, Buf0{}, c1, c2, c0);
        step(s + 5, Buf1{}, c2, c0, c1);
    }
    if (s < nk) step(s, Buf0{}, c0, c1, c2);
    if (s + 1 < nk) step(s + 1, Buf1{}, c1, c2, c0);
    if (s + 2 < nk) step(s + 2, Buf0{}, c2, c0, c1);
    if (s + 3 < nk) step(s + 3, Buf1{}, c0, c1, c2);
    if (s + 4 < nk) step(s + 4, Buf0{}, c1, c2, c0);
    __builtin_amdgcn_s_waitcnt(0);   // the last (clamped, unused) prefetches
    __syncthreads();

    if constexpr (R16 > 0) {
#pragma unroll
        for (int kk = 0; kk < kRp; kk += 16) {
            if (kk > 0) __syncthreads();      // the previous chunk has been read
            stage_t(kk);
            const bf16x8_t bl = load_lora_b(kk);
            __syncthreads();
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&thi[(32 * rt + j) * kTs + 8 * g]);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&tlo[(32 * rt + j) * kTs + 8 * g]);
                acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[rt], 0, 0, 0);
                acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bl, acc[rt], 0, 0, 0);
            }
        }
    }

    // epilogue: the bf16 tile through LDS 64 rows at a time, then 16-byte row stores.
    // Register e of tile rt holds C[32 rt + 8(e/4) + 4g + e%4][32 wave + j].
    const bool vec_ok = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(a.Y) % 16) == 0;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        uint16_t* cs = reinterpret_cast<uint16_t*>((pass & 1) ? xsB : xsA);
#pragma unroll
        for (int rt = 2 * pass; rt < 2 * pass + 2; ++rt) {
            const int col = 32 * wave + j;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * (rt - 2 * pass) + 8 * (e / 4) + 4 * g + (e % 4);
                cs[row * TN + col] = (uint16_t)(pack_bf16x2(acc[rt][e], 0.0f) & 0xFFFFu);
            }
        }
        // a bare barrier: the Y stores of the previous passes stay in flight (their LDS
        // reads, the only use of this buffer two passes ago, are complete)
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt untouched
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        for (int c = tid; c < (TM / 4) * (TN / 8); c += kThr) {
            const int row = c / (TN / 8), ch = c % (TN / 8);
            const int64_t gm = m0 + (TM / 4) * pass + row, gn = n0 + 8 * ch;
            if (gm >= M || gn >= N) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(&cs[row * TN + 8 * ch]);
            uint16_t* dst = a.Y + gm * N + gn;
            if (vec_ok && gn + 8 <= N) {
                *reinterpret_cast<uint4*>(dst) = v;
            } else {
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                for (int t = 0; t < 8 && gn + t < N; ++t) dst[t] = (uint16_t)(w4[t >> 1] >> ((t & 1) ? 16 : 0));
            }
        }
    }
}

// Partial LoRA products, T_p[m][j] = s * sum_{k in split p} X[m][k] A[k][j], in
// fp32, j < 16*R16 (columns >= r are 0).  Grid: (64-row groups, kSplits K
// splits); a workgroup's 4 waves take 16 rows each.  The split's A rows are
// transposed into LDS in chunks of up to kChunk 64-deep steps (one barrier pair
// per chunk), and each lane's X fragments stream from global memory into a ring
// of 4 register sets, loaded 4 steps ahead without conditions.  A chunk's step
// count is rounded up to a multiple of 4 with zero columns of A^T, whose X loads
// are clamped to the split's last step.  (An 8-deep ring measured slower.)  The GEMM
// kernel adds the kSplits partials of its rows in split order (deterministic)
// when it stages s X A.
// The pre-passes of one launch (a single call is a group of one): GEMM t owns the
// workgroups [blk0[t], blk0[t + 1]), one per 64-row block and K split (row block
// fastest), and writes its partials at T[t].
struct XaGroup {
    GemmArgs t[kMaxGemmGroup];
    float* T[kMaxGemmGroup];
    int32_t blk0[kMaxGemmGroup + 1];
    int32_t count;
};

template <int R16, bool kVec>
__global__ __launch_bounds__(256) void lora_xa_kernel(XaGroup gx) {
    // this workgroup's GEMM (uniform: a scalar search of the launch's prefix table)
    int task = 0;
    while (task + 1 < gx.count && (int32_t)blockIdx.x >= gx.blk0[task + 1]) ++task;
    const GemmArgs& a = gx.t[task];
    float* __restrict__ T = gx.T[task];
    const int32_t nrb = (int32_t)((a.M + 63) / 64);
    const int32_t local = (int32_t)blockIdx.x - gx.blk0[task];
    const int32_t rb = local % nrb;
    constexpr int kRp = 16 * R16;
    constexpr int kChunk = R16 == 1 ? 16 : (R16 == 2 ? 8 : 4);   // steps per A^T chunk (about 33 KB of LDS)
    constexpr int kS = kChunk * TK + 8;                           // A^T row pitch (elements)
    __shared__ __attribute__((aligned(16))) uint16_t at[kRp * kS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int64_t M = a.M, K = a.K;
    const int r = a.r;
    const int64_t nk = K / TK;
    const int split = local / nrb;
    const int64_t s0 = nk * split / kSplits, s1 = nk * (split + 1) / kSplits;
    const int64_t mrow = (int64_t)rb * 64 + 16 * wave + l16;
    const int64_t mrow_c = mrow < M ? mrow : M - 1;
    const uint16_t* xrow = a.X + mrow_c * K + 8 * q4;
    // kVec: r % 8 == 0 and A 16-byte aligned (A rows load as 16-byte pieces)
    constexpr bool a_vec = kVec;
    constexpr int cpr = kRp / 8;                                  // 16-byte chunks per A row (padded)
    constexpr int kAPer = kChunk * TK * cpr / 256;                // A pieces per thread and chunk

    floatx4_t acc[R16];
#pragma unroll
    for (int jt = 0; jt < R16; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jt][e] = 0.0f;

    // X fragments of step s (clamped to the split's last step): k = 64 s + 8 q4 + [0, 8)
    // and + 32
    auto load_xs = [&](int64_t s, uint4 (&d)[2]) {
        const int64_t sc = s < s1 ? s : s1 - 1;
        const uint4* p = reinterpret_cast<const uint4*>(xrow + sc * TK);
        d[0] = p[0];
        d[1] = p[4];
    };
    // A rows [64 c0, 64 c0 + 64 kChunk) transposed into at, in two parts (loads, then LDS
    // stores) so the loads can be issued before other loads; rows past the chunk's
    // nsteps steps and ranks >= r are zero
    auto issue_a = [&](int64_t c0, int nsteps, uint4 (&ar)[kAPer]) {
#pragma unroll
        for (int v = 0; v < kAPer; ++v) {
            const int c = tid + 256 * v;
            const int row = c / cpr, cc = c % cpr;
            const int64_t krow = c0 * TK + (row < nsteps * TK ? row : nsteps * TK - 1);
            const uint16_t* src = a.A + krow * r;
            if constexpr (a_vec) {
                ar[v] = *reinterpret_cast<const uint4*>(src + (cc * 8 < r ? cc * 8 : r - 8));
            } else {
                uint32_t e[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) e[t] = (uint32_t)src[cc * 8 + t < r ? cc * 8 + t : r - 1];
                ar[v] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
            }
        }
    };
    auto store_at = [&](int nsteps, const uint4 (&ar)[kAPer]) {
        if (a_vec && r == kRp) {
            // every 16-byte piece holds 8 live ranks: zero the piece once if its row is
            // past the chunk, then 8 two-byte stores with compile-time element indexes
#pragma unroll
            for (int v = 0; v < kAPer; ++v) {
                const int c = tid + 256 * v;
                const int row = c / cpr, cc = c % cpr;
                const bool live = row < nsteps * TK;
                const uint32_t w4[4] = {live ? ar[v].x : 0u, live ? ar[v].y : 0u, live ? ar[v].z : 0u,
                                        live ? ar[v].w : 0u};
#pragma unroll
                for (int t = 0; t < 8; ++t) at[(cc * 8 + t) * kS + row] = (uint16_t)(w4[t >> 1] >> ((t & 1) ? 16 : 0));
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < kAPer; ++v) {
            const int c = tid + 256 * v;
            const int row = c / cpr, cc = c % cpr;
            const bool live = row < nsteps * TK;
            const uint32_t w4[4] = {ar[v].x, ar[v].y, ar[v].z, ar[v].w};
            const int shift = (a_vec && cc * 8 + 8 > r) ? (cc * 8 - (r - 8)) : 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int st = t + shift;
                at[(cc * 8 + t) * kS + row] =
                    (live && cc * 8 + t < r && st < 8) ? (uint16_t)(w4[st >> 1] >> ((st & 1) ? 16 : 0)) : (uint16_t)0;
            }
        }
    };
    auto bare_barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) (LDS), vmcnt and expcnt untouched
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if (s0 < s1) {
        // the first chunk's A loads go first: the wait for them then leaves the X ring's
        // loads (issued after) in flight
        uint4 ar[kAPer];
        const int nsteps0 = (int)(s1 - s0 < kChunk ? s1 - s0 : kChunk);
        issue_a(s0, nsteps0, ar);
        uint4 xr[4][2];                       // ring: X of steps s .. s + 3 (slot = step % 4 from s0)
#pragma unroll
        for (int i = 0; i < 4; ++i) load_xs(s0 + i, xr[i]);
        store_at(nsteps0, ar);
        bare_barrier();
        auto one = [&](int64_t s, int kloc, uint4 (&xv)[2]) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, xv[kh]);
#pragma unroll
                for (int jt = 0; jt < R16; ++jt) {
                    const bf16x8_t ab =
                        *reinterpret_cast<const bf16x8_t*>(&at[(16 * jt + l16) * kS + kloc + 32 * kh + 8 * q4]);
                    acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ab, acc[jt], 0, 0, 0);
                }
            }
            load_xs(s + 4, xv);
        };
        for (int64_t c0 = s0; c0 < s1; c0 += kChunk) {
            const int nsteps = (int)(s1 - c0 < kChunk ? s1 - c0 : kChunk);
            if (c0 > s0) {
                bare_barrier();               // every wave is done with the previous chunk
                issue_a(c0, nsteps, ar);
                store_at(nsteps, ar);
                bare_barrier();
            }
            const int ngroups = (nsteps + 3) / 4;
            for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
                for (int i = 0; i < 4; ++i) one(c0 + 4 * gi + i, (4 * gi + i) * TK, xr[i]);
            }
        }
    }
    // 16x16 output: lane holds C[4 q4 + e][l16]
    float* Tp = T + (int64_t)split * M * kRp;
#pragma unroll
    for (int jt = 0; jt < R16; ++jt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = (int64_t)rb * 64 + 16 * wave + 4 * q4 + e;
            if (m < M) Tp[m * kRp + 16 * jt + l16] = acc[jt][e] * a.lora_scale;
        }
    }
}

}  // namespace v4

template <bool kNested>
void launch_fast_r(const v4::GemmGroup& g, hipStream_t s, int r16) {
    const dim3 grid((unsigned)g.tile0[g.count]), block(512);
    switch (r16) {
        case 0: hipLaunchKernelGGL((v4::gemm_fast_kernel<0, kNested>), grid, block, 0, s, g); break;
        case 1: hipLaunchKernelGGL((v4::gemm_fast_kernel<1, kNested>), grid, block, 0, s, g); break;
        case 2: hipLaunchKernelGGL((v4::gemm_fast_kernel<2, kNested>), grid, block, 0, s, g); break;
        case 3: hipLaunchKernelGGL((v4::gemm_fast_kernel<3, kNested>), grid, block, 0, s, g); break;
        default: hipLaunchKernelGGL((v4::gemm_fast_kernel<4, kNested>), grid, block, 0, s, g); break;
    }
}

// an adapter whose rows load as 16-byte pieces
bool lora_vec(const GemmArgs& a) { return (a.r % 8) == 0 && (reinterpret_cast<uintptr_t>(a.A) % 16) == 0; }

int64_t fast_tiles(const GemmArgs& a) { return ((a.N + v4::TN - 1) / v4::TN) * ((a.M + v4::TM - 1) / v4::TM); }

// pre-passes that share the rank class and the 16-byte adapter loads, in one launch
void launch_lora_xa_group(const GemmArgs* const* as, float* const* Ts, int32_t count, hipStream_t s) {
    v4::XaGroup g;
    std::memset(&g, 0, sizeof(g));
    int64_t blocks = 0;
    for (int32_t i = 0; i < count; ++i) {
        g.t[i] = *as[i];
        g.T[i] = Ts[i];
        g.blk0[i] = (int32_t)blocks;
        blocks += ((as[i]->M + 63) / 64) * v4::kSplits;
    }
    g.blk0[count] = (int32_t)blocks;
    g.count = count;
    const dim3 grid((unsigned)blocks);
    const bool vec = lora_vec(*as[0]);
    const int r16 = (as[0]->r + 15) / 16;
#define QK_LORA_XA(R)                                                                  \
    do {                                                                               \
        if (vec) hipLaunchKernelGGL((v4::lora_xa_kernel<R, true>), grid, dim3(256), 0, s, g); \
        else hipLaunchKernelGGL((v4::lora_xa_kernel<R, false>), grid, dim3(256), 0, s, g);    \
    } while (0)
    switch (r16) {
        case 1: QK_LORA_XA(1); break;
        case 2: QK_LORA_XA(2); break;
        case 3: QK_LORA_XA(3); break;
        default: QK_LORA_XA(4); break;
    }
#undef QK_LORA_XA
}

void launch_lora_xa(const GemmArgs& a, float* T, hipStream_t s, int r16) {
    (void)r16;
    const GemmArgs* as[1] = {&a};
    float* Ts[1] = {T};
    launch_lora_xa_group(as, Ts, 1, s);
}

// GEMMs that share the LoRA rank class and the nesting, in one launch (their LoRA
// partials already formed, task t's at Ts[t]): the tiles of all tasks, task by task in
// the given order.
hipError_t launch_fast_group(const GemmArgs* const* as, float* const* Ts, int32_t count, hipStream_t s) {
    v4::GemmGroup g;
    std::memset(&g, 0, sizeof(g));
    const int r16 = as[0]->A ? (as[0]->r + 15) / 16 : 0;
    int64_t tiles = 0;
    for (int32_t i = 0; i < count; ++i) {
        g.t[i] = *as[i];
        g.T[i] = Ts[i];
        g.tile0[i] = (int32_t)tiles;
        tiles += fast_tiles(*as[i]);
    }
    g.tile0[count] = (int32_t)tiles;
    g.count = count;
    if (g.t[0].w.nested) launch_fast_r<true>(g, s, r16);
    else launch_fast_r<false>(g, s, r16);
    return hipGetLastError();
}

hipError_t launch_fast(const GemmArgs& a, void* workspace, hipStream_t s) {
    float* T = reinterpret_cast<float*>(workspace);
    if (a.A) {
        launch_lora_xa(a, T, s, (a.r + 15) / 16);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const GemmArgs* as[1] = {&a};
    float* Ts[1] = {T};
    return launch_fast_group(as, Ts, 1, s);
}

// Ts[i] = T_0[i] + ... + T_{kSplits-1}[i], split order (the same order the GEMM uses).
__global__ __launch_bounds__(256) void lora_split_sum_kernel(const float* __restrict__ T, int64_t n, float* __restrict__ Ts) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = T[i];
    for (int p = 1; p < v4::kSplits; ++p) acc += T[(int64_t)p * n + i];
    Ts[i] = acc;
}

}  // namespace

hipError_t launch_lora_xa_sum(const void* X, int64_t M, int64_t K, const void* A, int32_t r, float lora_scale,
                              float* T_splits, float* Ts, hipStream_t s) {
    GemmArgs a{};
    a.X = reinterpret_cast<const uint16_t*>(X);
    a.A = reinterpret_cast<const uint16_t*>(A);
    a.M = M;
    a.K = K;
    a.r = r;
    a.lora_scale = lora_scale;
    const int r16 = (r + 15) / 16;
    launch_lora_xa(a, T_splits, s, r16);
    const int64_t n = M * 16 * r16;
    hipLaunchKernelGGL(lora_split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T_splits, n, Ts);
    return hipGetLastError();
}

// Scratch of qk_gemm_nf4_noalloc: the LoRA pre-pass partials live in this
// file-scope device array instead of a caller workspace.  Each device holds its
// own copy (at its own address) until the process ends; every call on a device
// shares it, so calls that overlap on one device race.  The pre-pass writes every
// partial it leaves for the GEMM, so nothing has to be cleared between calls.
// Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): it passes the device address that hipGetSymbolAddress
// returns, looked up once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

size_t gemm_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t gemm_noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t gemm_workspace_bytes(int64_t M, int32_t r) {
    return r > 0 ? (size_t)v4::kSplits * (size_t)M * (size_t)(((r + 15) / 16) * 16) * sizeof(float) : 0;
}

namespace {

GemmArgs gemm_args(const void* X, int64_t M, const MatArgs& w, const void* A, const void* B, int32_t r,
                   float lora_scale, void* Y) {
    GemmArgs a;
    a.X = reinterpret_cast<const uint16_t*>(X);
    a.A = reinterpret_cast<const uint16_t*>(A);
    a.B = reinterpret_cast<const uint16_t*>(B);
    a.Y = reinterpret_cast<uint16_t*>(Y);
    a.w = w.w;
    a.M = M;
    a.N = w.N;
    a.K = w.K;
    a.r = A ? r : 0;
    a.lora_scale = lora_scale;
    return a;
}

// the fast path's buffer offsets of a 256-row X tile are 32-bit: 256 * K * 2 < 2^31
bool fast_ok(const GemmArgs& a) {
    return (a.K % BK) == 0 && (a.K % a.w.blocksize) == 0 && (reinterpret_cast<uintptr_t>(a.X) % 16) == 0 &&
           (reinterpret_cast<uintptr_t>(a.w.codes) % 16) == 0 && a.K < ((int64_t)1 << 22);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

hipError_t launch_gemm(const void* X, int64_t M, const MatArgs& w, const void* A, const void* B, int32_t r,
                       float lora_scale, void* Y, void* workspace, hipStream_t s, const char** variant) {
    const GemmArgs a = gemm_args(X, M, w, A, B, r, lora_scale, Y);
    if (a.M > 65535LL * BM || a.N > 65535LL * BN) return hipErrorInvalidValue;   // grid limits of both paths
    if (fast_ok(a)) {
        *variant = "mfma 32x32x16 bf16, 256x256x64 tiles, W dequantized into B fragments, LoRA X*A pre-pass + epilogue";
        return launch_fast(a, workspace, s);
    }
    // the vectorized generic loads use 32-bit byte offsets within a 128-row tile
    if (w.K < ((int64_t)1 << 22)) {
        *variant = "generic (16-byte loads realigned, flat-index block scales), 128x128x64 tiles";
        return launch_typed<true, true>(a, s);
    }
    *variant = "generic (element loads, flat-index dequantization), 128x128x64 tiles";
    return launch_typed<true, false>(a, s);
}

size_t gemm_group_workspace_bytes(const GemmItem* items, int32_t count) {
    size_t b = 0;
    for (int32_t i = 0; i < count; ++i)
        if (items[i].A) b += align256(gemm_workspace_bytes(items[i].M, items[i].r));
    return b;
}

hipError_t launch_gemm_group(const GemmItem* items, int32_t count, void* workspace, hipStream_t s,
                             const char** variant) {
    // each task with an adapter owns a slice of the workspace, in task order
    std::vector<GemmArgs> args(count);
    std::vector<float*> ts(count, nullptr);
    size_t off = 0;
    for (int32_t i = 0; i < count; ++i) {
        const GemmItem& it = items[i];
        args[i] = gemm_args(it.X, it.M, it.w, it.A, it.B, it.r, it.lora_scale, it.Y);
        if (args[i].M > 65535LL * BM || args[i].N > 65535LL * BN) return hipErrorInvalidValue;
        if (it.A) {
            ts[i] = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + off);
            off += align256(gemm_workspace_bytes(it.M, it.r));
        }
    }
    // tasks the fast kernel cannot take go one by one; the others are launched together
    // by rank class and nesting, the longest rows first (their tiles take longest, so
    // they start first and the shorter ones fill in behind them), at most kMaxGemmGroup
    // at a time
    std::vector<int32_t> fast;
    for (int32_t i = 0; i < count; ++i) {
        if (fast_ok(args[i])) {
            fast.push_back(i);
            continue;
        }
        const char* v = nullptr;
        const hipError_t e = launch_gemm(items[i].X, items[i].M, items[i].w, items[i].A, items[i].B, items[i].r,
                                         items[i].lora_scale, items[i].Y, ts[i], s, &v);
        if (e != hipSuccess) return e;
        *variant = v;
    }
    // the LoRA pre-passes of the fast GEMMs, together by rank class and adapter loads
    // (their latency chains overlap: one launch instead of one per GEMM)
    {
        std::vector<bool> done(count, false);
        for (size_t f = 0; f < fast.size(); ++f) {
            const int32_t i0 = fast[f];
            if (done[i0] || !args[i0].A) continue;
            const int r16 = (args[i0].r + 15) / 16;
            const bool vec = lora_vec(args[i0]);
            const GemmArgs* as[kMaxGemmGroup];
            float* tsg[kMaxGemmGroup];
            int32_t n = 0;
            int64_t blocks = 0;
            for (size_t f2 = f; f2 < fast.size() && n < kMaxGemmGroup; ++f2) {
                const int32_t i = fast[f2];
                if (done[i] || !args[i].A || (args[i].r + 15) / 16 != r16 || lora_vec(args[i]) != vec) continue;
                const int64_t b = ((args[i].M + 63) / 64) * v4::kSplits;
                if (blocks + b > ((int64_t)1 << 31) - 1) continue;
                as[n] = &args[i];
                tsg[n] = ts[i];
                blocks += b;
                ++n;
                done[i] = true;
            }
            launch_lora_xa_group(as, tsg, n, s);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    std::stable_sort(fast.begin(), fast.end(), [&](int32_t x, int32_t y) { return args[x].K > args[y].K; });
    std::vector<bool> used(count, false);
    for (size_t f = 0; f < fast.size(); ++f) {
        const int32_t i0 = fast[f];
        if (used[i0]) continue;
        const int r16 = args[i0].A ? (args[i0].r + 15) / 16 : 0;
        const bool nested = args[i0].w.nested != 0;
        const GemmArgs* as[kMaxGemmGroup];
        float* tsg[kMaxGemmGroup];
        int32_t n = 0;
        int64_t tiles = 0;
        for (size_t f2 = f; f2 < fast.size() && n < kMaxGemmGroup; ++f2) {
            const int32_t i = fast[f2];
            if (used[i] || (args[i].A ? (args[i].r + 15) / 16 : 0) != r16 || (args[i].w.nested != 0) != nested) continue;
            if (tiles + fast_tiles(args[i]) > ((int64_t)1 << 31) - 1) continue;
            as[n] = &args[i];
            tsg[n] = ts[i];
            tiles += fast_tiles(args[i]);
            ++n;
            used[i] = true;
        }
        const hipError_t e = launch_fast_group(as, tsg, n, s);
        if (e != hipSuccess) return e;
        *variant = "mfma 32x32x16 bf16, 256x256x64 tiles of the group's GEMMs in one launch, W dequantized into B "
                   "fragments, LoRA X*A pre-pass per GEMM + epilogue";
    }
    return hipSuccess;
}

}  // namespace qk
