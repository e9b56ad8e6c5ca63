// Prefill / training GEMM of a frozen 4-bit base layer with an unmerged LoRA
// adapter, for gfx950:
//     Y = X · deq(W)^T + s · (X · A) · B
// "LLM 相關知識" (technicalnotes, tag qlora), sections 2-2 LoRA (W + ΔW with
// ΔW = A × B, A and B trainable BF16), 5 動態反量化 (the 4-bit base is restored to
// BF16 tile by tile just before the matmul) and 8 (without merging, base output
// and LoRA output are computed separately and added);
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 (QLoRA forward).
//
// Structure (one workgroup per BM x BN output tile, 4 waves as 2 x 2, each wave
// 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_bf16):
//   * K loop in steps of 64 with two LDS buffers.  The X tile is copied to LDS
//     with 16-byte loads; the W tile is dequantized by the workgroup on the way
//     into LDS: each thread takes 32 weights of one row (16 code bytes, one
//     block), computes bf16(RN(level * a')) exactly as the dequantize kernel does
//     and writes 64 bytes of bf16.  The next step's global loads are issued
//     before the current step's MFMAs so they overlap.
//   * LDS rows are padded to 144 bytes so the 16-byte fragment reads of 8
//     consecutive rows fall in distinct banks.
//   * LoRA: T = X · A (fp32, [BM, r]) accumulates in the same K loop from the X
//     tile already in LDS (each wave owns 32 rows of T; v_mfma_f32_16x16x32_bf16);
//     after the loop s*T is split into bf16 hi + lo parts and (s T) · B is added
//     to the accumulators with two more MFMAs per tile.
//   * Epilogue: fp32 accumulators -> bf16 (RNE) -> Y.
// A generic variant (template flag) loads X element by element and dequantizes
// W with flat indexing, for K that is not a multiple of 64 or of the block size
// (blocks straddling rows) and unaligned X.
#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kLdsStride = BK + 8;        // bf16 elements per LDS row (144 bytes)
constexpr int kMaxRank = 64;

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

template <bool kGeneric, bool kLora>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
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
    uint16_t xg[kGeneric ? 32 : 1];   // generic path: 32 X elements per thread
    uint32_t cg[kGeneric ? 16 : 1];   // generic path: 16 packed code bytes (re-packed)
    float scg[kGeneric ? 32 : 1];
    constexpr int kAPer = kLora ? kMaxRank * BK / kThreads : 1;   // 16
    uint16_t ag[kAPer];               // LoRA A^T elements owned by this thread

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
                csc = wscale(a.w, e0 / a.w.blocksize);
            } else {
                cr = make_uint4(0, 0, 0, 0);
                csc = 0.0f;
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
                    sc = wscale(a.w, e / a.w.blocksize);
                }
                cg[i >> 1] |= code << ((i & 1) ? 0 : 4);
                scg[i] = sc;
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

template <bool kGeneric>
hipError_t launch_typed(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    if (a.A)
        hipLaunchKernelGGL((gemm_kernel<kGeneric, true>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_kernel<kGeneric, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* X, int64_t M, const MatArgs& w, const void* A, const void* B, int32_t r,
                       float lora_scale, void* Y, hipStream_t s, const char** variant) {
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
    if (a.M > 65535LL * BM) return hipErrorInvalidValue;
    const bool fast = (w.K % BK) == 0 && (w.K % w.w.blocksize) == 0 && (reinterpret_cast<uintptr_t>(X) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(w.w.codes) % 16) == 0;
    if (fast) {
        *variant = "mfma 32x32x16 bf16, 128x128x64 tiles, W dequantized into LDS, LoRA in the K loop";
        return launch_typed<false>(a, s);
    }
    *variant = "generic (element loads, flat-index dequantization), 128x128x64 tiles";
    return launch_typed<true>(a, s);
}

}  // namespace qk
