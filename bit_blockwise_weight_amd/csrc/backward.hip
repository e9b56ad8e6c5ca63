// QLoRA backward of a frozen 4-bit base layer with a LoRA adapter, for gfx950.
//
// Forward: Y = X · deq(W)^T + s · (X · A) · B   (W [N, K] frozen, A [K, r], B [r, N]).
// "Tim Dettmers 如何用 bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？", section "QLoRA 把
// frozen 4-bit base 與可訓練 adapter 分開": the 4-bit base is dequantized to the
// compute dtype in the backward pass as in the forward and stays frozen; only the
// adapter is trained, so the gradients are the input's and the adapter's.
// "LLM 相關知識" (technicalnotes, tag qlora), section 4: the INT4 base is frozen
// and the BF16 matrices A and B train.
// Gradients for an upstream dY [M, N]:
//     G  = dY · B^T                          [M, r]
//     dX = dY · deq(W) + s · G · A^T         [M, K]   (bf16 out)
//     dA = s · X^T · G                       [K, r]   (fp32 out)
//     dB = s · (X · A)^T · dY                [r, N]   (fp32 out)
//
// dX: 128 x 128 output tiles (rows of dY, columns k of W), reduction over n in
// steps of 64, 4 waves as 2 x 2, each 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16
// tiles.  W is used untransposed here, so its tile is dequantized by the workgroup
// into LDS as W^T: thread t reads 8 rows x 4 columns of codes (4 nibbles per row),
// computes bf16(RN(level * a')) exactly as qk_dequantize does, and writes each
// column's 8 values (8 consecutive n) as one 16-byte LDS store.  The LoRA term:
// s·G comes from a pre-pass (the MFMA kernel of the forward's s·X·A, run on dY
// and B^T), is split into bf16 hi + lo in the epilogue and multiplied by A^T.
// dA and dB are reductions over the M token rows with r outputs per column: a
// VALU kernel takes 256 columns x one slice of rows per workgroup (fp32 FMAs, rows
// in increasing order) and writes per-slice partials, which a second kernel adds
// in slice order (deterministic).
#include <type_traits>

#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;                  // dY / dX rows per tile
constexpr int BN = 128;                  // k columns of dX per tile
constexpr int BK = 64;                   // n per reduction step
constexpr int kThreads = 256;
constexpr int kStride = BK + 8;          // bf16 per LDS row (144 bytes)
constexpr int kMaxRank = 64;
constexpr int kSlices = 16;              // row slices of the dA / dB reductions

struct DxArgs {
    const uint16_t* dY;   // [M, N]
    DeqArgs w;            // W [N, K]
    const uint16_t* A;    // [K, r] or null
    uint16_t* dX;         // [M, K]
    const float* Gs;      // [M, rpad]: s * dY B^T (fp32, ranks >= r zero)
    int64_t M, N, K;
    int32_t r;
};

__device__ __forceinline__ float block_scale(const DeqArgs& a, int64_t blk) {
    if (!a.nested) return a.absmax[blk];
    return __fadd_rn(__fmul_rn((float)a.q8[blk], a.dq_scale[blk / QK_DQ_BLOCK]), *a.dq_mean);
}

template <bool kLora>
__global__ __launch_bounds__(kThreads) void dx_kernel(DxArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ys[2][BM * kStride];
    __shared__ __attribute__((aligned(16))) uint16_t wt[2][BN * kStride];
    __shared__ float lev[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t k0 = (int64_t)blockIdx.x * BN;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int rpad = kLora ? ((a.r + 15) / 16) * 16 : 0;
    if (tid < 16) lev[tid] = a.w.levels[tid];
    const int64_t nsteps = N / BK;

    // W^T staging: thread takes rows n = step*64 + 8*(t / 32) + i (i < 8), columns k = k0 + 4*(t % 32) .. +4
    const int rg = tid >> 5, kq = tid & 31;
    const int64_t wk = k0 + 4 * kq;
    const bool wk_ok = wk < K;               // K % 4 == 0: the 4 columns are all in range or all out

    uint4 yr[4];
    uint32_t cw[8];
    float sc[8];
    auto load_step = [&](int64_t st) {
        const int64_t n0 = st * BK;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = tid + kThreads * v;
            const int row = c >> 3, ch = c & 7;
            const int64_t gm = m0 + row;
            yr[v] = gm < M ? *reinterpret_cast<const uint4*>(a.dY + gm * N + n0 + ch * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t e = (n0 + 8 * rg + i) * K + wk;       // even: 2 code bytes, one block
            cw[i] = wk_ok ? (uint32_t)*reinterpret_cast<const uint16_t*>(a.w.codes + e / 2) : 0u;
            sc[i] = wk_ok ? block_scale(a.w, e >> a.w.blocksize_log2) : 0.0f;
        }
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = tid + kThreads * v;
            const int row = c >> 3, ch = c & 7;
            *reinterpret_cast<uint4*>(&ys[buf][row * kStride + ch * 8]) = yr[v];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // column c: code byte c / 2, high nibble first
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t sh = 8 * (c >> 1) + ((c & 1) ? 0 : 4);
                const float y0 = __fmul_rn(lev[(cw[i] >> sh) & 0xFu], sc[i]);
                const float y1 = __fmul_rn(lev[(cw[i + 1] >> sh) & 0xFu], sc[i + 1]);
                o[i >> 1] = pack_bf16x2(y0, y1);
            }
            *reinterpret_cast<uint4*>(&wt[buf][(4 * kq + c) * kStride + 8 * rg]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };

    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    __syncthreads();   // lev ready
    load_step(0);
    store_step(0);
    __syncthreads();

    const int fi = lane & 31;         // fragment row / column within a 32 tile
    const int fg = lane >> 5;         // 8-element half of a 16-deep MFMA step
    for (int64_t st = 0; st < nsteps; ++st) {
        const int buf = (int)(st & 1);
        if (st + 1 < nsteps) load_step(st + 1);
        const uint16_t* yb = ys[buf];
        const uint16_t* wb = wt[buf];
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(&yb[(wm * 64 + i * 32 + fi) * kStride + kk + 8 * fg]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&wb[(wn * 64 + j * 32 + fi) * kStride + kk + 8 * fg]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (st + 1 < nsteps) {
            store_step(buf ^ 1);
            __syncthreads();
        }
    }

    if constexpr (kLora) {
        // s*G rows of this tile -> LDS as bf16 hi / lo in ys[0] / ys[1] (hi + lo = s*G to 2^-16)
        uint16_t* ghi = ys[0];
        uint16_t* glo = ys[1];
        for (int e = tid; e < BM * rpad; e += kThreads) {
            const int row = e / rpad, col = e % rpad;
            const float v = m0 + row < M ? a.Gs[(m0 + row) * rpad + col] : 0.0f;
            const uint32_t hb = pack_bf16x2(v, 0.0f) & 0xFFFFu;
            const float h = as_float(hb << 16);
            ghi[row * kStride + col] = (uint16_t)hb;
            glo[row * kStride + col] = (uint16_t)(pack_bf16x2(v - h, 0.0f) & 0xFFFFu);
        }
        // A^T tile: wt[0][col][j] = A[k0 + col][j]
        for (int e = tid; e < BN * rpad; e += kThreads) {
            const int col = e / rpad, j = e % rpad;
            const int64_t gk = k0 + col;
            wt[0][col * kStride + j] = (j < a.r && gk < K) ? a.A[gk * a.r + j] : (uint16_t)0;
        }
        __syncthreads();
        for (int kk = 0; kk < rpad; kk += 16) {
            bf16x8_t ah[2], al[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + fi;
                ah[i] = *reinterpret_cast<const bf16x8_t*>(&ghi[row * kStride + kk + 8 * fg]);
                al[i] = *reinterpret_cast<const bf16x8_t*>(&glo[row * kStride + kk + 8 * fg]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&wt[0][(wn * 64 + j * 32 + fi) * kStride + kk + 8 * fg]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bfr[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bfr[j], acc[i][j], 0, 0, 0);
                }
        }
    }

    // epilogue: lane holds C[8b + 4 (l / 32) + q][l % 32] in register 4b + q
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t gk = k0 + wn * 64 + j * 32 + fi;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 8 * (e / 4) + 4 * fg + (e % 4);
                const int64_t gm = m0 + wm * 64 + i * 32 + row;
                if (gm < M && gk < K) a.dX[gm * K + gk] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
            }
        }
    }
}

// Partial reductions over a slice of the M rows: part[slice][l][j] = sum over rows m
// of the slice, increasing, of P[m][l] * Q[m][j] (P bf16 [M, L], Q fp32 [M, rpad]).
// Thread t of workgroup (bx, slice) owns column l = 256 bx + t and all rpad j.
template <int R16>
__global__ __launch_bounds__(256) void tn_partial_kernel(const uint16_t* __restrict__ P, int64_t L,
                                                         const float* __restrict__ Q, int64_t M,
                                                         float* __restrict__ part) {
    constexpr int kRp = 16 * R16;
    constexpr int kRows = 64;
    __shared__ float qs[kRows][kRp];
    const int tid = threadIdx.x;
    const int64_t l = (int64_t)blockIdx.x * 256 + tid;
    const int slice = blockIdx.y;
    const int64_t r0 = M * slice / kSlices, r1 = M * (slice + 1) / kSlices;
    float acc[kRp];
#pragma unroll
    for (int j = 0; j < kRp; ++j) acc[j] = 0.0f;
    for (int64_t mb = r0; mb < r1; mb += kRows) {
        const int nrows = (int)(r1 - mb < kRows ? r1 - mb : kRows);
        __syncthreads();
        for (int e = tid; e < nrows * kRp; e += 256) qs[e / kRp][e % kRp] = Q[(mb + e / kRp) * kRp + e % kRp];
        __syncthreads();
        if (l < L) {
            for (int i = 0; i < nrows; ++i) {
                const float p = as_float((uint32_t)P[(mb + i) * L + l] << 16);
#pragma unroll
                for (int j = 0; j < kRp; ++j) acc[j] = __builtin_fmaf(p, qs[i][j], acc[j]);
            }
        }
    }
    if (l < L) {
#pragma unroll
        for (int j = 0; j < kRp; ++j) part[((int64_t)slice * L + l) * kRp + j] = acc[j];
    }
}

// out = sum of the slices in slice order; transposed: out[j][l] (dB), else out[l][j] (dA).
__global__ __launch_bounds__(256) void tn_reduce_kernel(const float* __restrict__ part, int64_t L, int32_t rpad,
                                                        int32_t r, float* __restrict__ out, int32_t transposed) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= L * r) return;
    const int64_t l = e / r;
    const int j = (int)(e % r);
    float v = part[l * rpad + j];
    for (int sl = 1; sl < kSlices; ++sl) v += part[((int64_t)sl * L + l) * rpad + j];
    if (transposed) out[(int64_t)j * L + l] = v;
    else out[l * r + j] = v;
}

hipError_t launch_tn(const uint16_t* P, int64_t L, const float* Q, int64_t M, int32_t r, float* part, float* out,
                     bool transposed, hipStream_t s) {
    const int r16 = (r + 15) / 16;
    const dim3 grid((unsigned)((L + 255) / 256), kSlices);
    switch (r16) {
        case 1: hipLaunchKernelGGL(tn_partial_kernel<1>, grid, dim3(256), 0, s, P, L, Q, M, part); break;
        case 2: hipLaunchKernelGGL(tn_partial_kernel<2>, grid, dim3(256), 0, s, P, L, Q, M, part); break;
        case 3: hipLaunchKernelGGL(tn_partial_kernel<3>, grid, dim3(256), 0, s, P, L, Q, M, part); break;
        default: hipLaunchKernelGGL(tn_partial_kernel<4>, grid, dim3(256), 0, s, P, L, Q, M, part); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tn_reduce_kernel, dim3((unsigned)((L * r + 255) / 256)), dim3(256), 0, s, part, L,
                       16 * r16, r, out, transposed ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

// B [r, N] -> Bt [N, r] (bf16), so that s dY B^T has the layout of the forward's s X A.
__global__ __launch_bounds__(256) void transpose_b_kernel(const uint16_t* __restrict__ B, int64_t N, int32_t r,
                                                          uint16_t* __restrict__ Bt) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= N * r) return;
    const int64_t n = e / r;
    const int j = (int)(e % r);
    Bt[e] = B[(int64_t)j * N + n];
}

// workspace: T splits [8][M][rpad] | Ts [M][rpad] | Gs [M][rpad] | partials [kSlices][max(N, K)][rpad] (fp32)
//            | Bt [N][r] (bf16)
size_t qlora_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (r <= 0) return 0;
    const size_t rpad = (size_t)((r + 15) / 16) * 16;
    const size_t L = (size_t)(N > K ? N : K);
    return gemm_workspace_bytes(M, r) + 2 * (size_t)M * rpad * sizeof(float) +
           (size_t)kSlices * L * rpad * sizeof(float) + (size_t)N * rpad * sizeof(uint16_t);
}

hipError_t launch_qlora_backward(const void* dY, int64_t M, const MatArgs& w, const void* X, const void* A,
                                 const void* B, int32_t r, float lora_scale, void* dX, float* dA, float* dB,
                                 void* workspace, hipStream_t s) {
    const bool lora = A != nullptr;
    const int64_t N = w.N, K = w.K;
    const size_t rpad = lora ? (size_t)((r + 15) / 16) * 16 : 0;
    char* ws = reinterpret_cast<char*>(workspace);
    float* Tsplit = reinterpret_cast<float*>(ws);
    float* Ts = lora ? reinterpret_cast<float*>(ws + gemm_workspace_bytes(M, r)) : nullptr;
    float* Gs = lora ? Ts + (size_t)M * rpad : nullptr;
    float* part = lora ? Gs + (size_t)M * rpad : nullptr;
    uint16_t* Bt = lora ? reinterpret_cast<uint16_t*>(part + (size_t)kSlices * (N > K ? N : K) * rpad) : nullptr;
    hipError_t e = hipSuccess;
    if (lora) {
        // s G = s dY B^T first: the dX epilogue and dA read it
        hipLaunchKernelGGL(transpose_b_kernel, dim3((unsigned)((N * r + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const uint16_t*>(B), N, r, Bt);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_lora_xa_sum(dY, M, N, Bt, r, lora_scale, Tsplit, Gs, s);
        if (e != hipSuccess) return e;
    }

    DxArgs a;
    a.dY = reinterpret_cast<const uint16_t*>(dY);
    a.w = w.w;
    a.A = reinterpret_cast<const uint16_t*>(A);
    a.dX = reinterpret_cast<uint16_t*>(dX);
    a.Gs = Gs;
    a.M = M;
    a.N = N;
    a.K = K;
    a.r = lora ? r : 0;
    const int64_t gy = (M + BM - 1) / BM;
    if (gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((K + BN - 1) / BN), (unsigned)gy);
    if (lora) hipLaunchKernelGGL(dx_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(dx_kernel<false>, grid, dim3(kThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || !lora) return e;
    // dA = X^T (s G): columns l = k of X
    e = launch_tn(reinterpret_cast<const uint16_t*>(X), K, Gs, M, r, part, dA, false, s);
    if (e != hipSuccess) return e;
    // dB = (s X A)^T dY: Ts = s X A, columns l = n of dY, stored transposed [r][N]
    e = launch_lora_xa_sum(X, M, K, A, r, lora_scale, Tsplit, Ts, s);
    if (e != hipSuccess) return e;
    return launch_tn(reinterpret_cast<const uint16_t*>(dY), N, Ts, M, r, part, dB, true, s);
}

}  // namespace qk
