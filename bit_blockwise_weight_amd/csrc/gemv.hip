// Decode-time GEMV with the dequantized weight, for gfx950:
//     y[m, n] = sum_k x[m, k] * deq(W)[n, k],   m < M <= 16
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 【代码】 (the 4-bit linear
// layer's forward is dequantize + matmul); "Tim Dettmers 如何用 bitsandbytes 與
// QLoRA 降低 LLM 訓練門檻？", section on speed (unpacking and dequantizing must be
// fused, or 4-bit can be slower than 16-bit).  The weight is never written out.
//
// Fast path (K a multiple of 64 and of the block size):
//   * A workgroup owns a tile of 32 weight rows; its S waves split K in
//     interleaved steps of 64 (wave w takes steps w, w+S, ...), so at any time
//     the waves of a workgroup read neighbouring bytes of each row.
//   * In a step, lane l (row j = l % 32 of the tile, half g = l / 32) loads the
//     16 code bytes of weights [64s + 32g, 64s + 32g + 32) of its row: the two
//     lanes of a row read one 32-byte run, and one step of a row lies inside one
//     absmax block.
//   * Decoding: an LDS table maps a code byte to the pair (bf16 level of the high
//     nibble, bf16 level of the low nibble) as one dword, replicated 64 times and
//     interleaved so that lane l reads copy l: the address (byte << 8 | 4l) is
//     one v_perm, the read never conflicts.
//   * Four v_mfma_f32_32x32x16_bf16 per step: B = the lane's 8 weights of that
//     MFMA, A = x[i = l % 32][same 8 k] (rows i >= M are zero).  The step's
//     32 x 32 partial is multiplied by the row's block scale a' (fp32) and added
//     to the accumulator, so the scale costs one FMA per kept output register
//     per step instead of one multiply per weight.
//   * The S partial tiles are summed through LDS in a fixed order (deterministic).
// The levels are used as bf16 and the block scale is applied in fp32 after the
// bf16 products; the result agrees with the fp64 product on the bf16-dequantized
// weight within the documented tolerance.
//
// Generic path (any K, blocks straddling rows): one wave per row, each lane walks
// k = lane, lane + 64, ... and dequantizes each weight exactly as the dequantize
// kernel does (bf16 of level * a'), with fp32 accumulation.
#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;          // rows per tile (MFMA 32x32)
constexpr int kStep = 64;          // k per step
constexpr int kTabCopies = 64;

struct GemvArgs {
    const uint16_t* x;   // [M, K] bf16 bits
    uint16_t* y;         // [M, N] bf16 bits
    DeqArgs w;
    int64_t N;
    int64_t K;
    int32_t M;
};

__device__ __forceinline__ float row_scale(const DeqArgs& a, int64_t blk) {
    if (!a.nested) return a.absmax[blk];
    return __fadd_rn(__fmul_rn((float)a.q8[blk], a.dq_scale[blk / QK_DQ_BLOCK]), *a.dq_mean);
}

// Fill the byte -> (bf16 level hi nibble | bf16 level lo nibble << 16) table, 64 copies.
__device__ __forceinline__ void fill_pair_table(uint32_t* tab, const float* levels, int nthreads) {
    for (int i = threadIdx.x; i < 256 * kTabCopies; i += nthreads) {
        const int b = i / kTabCopies;
        tab[i] = pack_bf16x2(levels[b >> 4], levels[b & 15]);
    }
}

// MB = number of 8-row groups of the 32x32 output that hold real rows (M <= 8*MB)
template <int MB, int S>
__global__ __launch_bounds__(S * 64) void gemv_mfma_kernel(GemvArgs a) {
    extern __shared__ uint32_t lds[];          // 64 KB pair table, reused for the reduction
    fill_pair_table(lds, a.w.levels, S * 64);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 31;                   // row of the tile / column of the MFMA output
    const int g = lane >> 5;                   // which 32-weight half of the step
    const int64_t n = (int64_t)blockIdx.x * kRows + j;
    const bool row_ok = n < a.N;
    const int64_t K = a.K;
    const int64_t nsteps = K / kStep;
    const int M = a.M;
    const uint8_t* row_codes = a.w.codes + (row_ok ? n : 0) * (K / 2);
    const int64_t row_elem0 = (row_ok ? n : 0) * K;
    const uint32_t lane_sel = (uint32_t)lane * 4u;         // low byte of the LDS address
    const char* tab = reinterpret_cast<const char*>(lds);
    const int xi = lane & 31;                                // x row held by this lane
    const bool x_ok = xi < M;
    const uint16_t* xrow = a.x + (int64_t)(x_ok ? xi : 0) * K;

    floatx16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    for (int64_t s = wave; s < nsteps; s += S) {
        const int64_t k0 = s * kStep + g * 32;
        uint4 cw = make_uint4(0, 0, 0, 0);
        if (row_ok) cw = *reinterpret_cast<const uint4*>(row_codes + k0 / 2);
        uint4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[q] = x_ok ? *reinterpret_cast<const uint4*>(xrow + k0 + 8 * q) : make_uint4(0, 0, 0, 0);
        }
        const float sc = row_ok ? row_scale(a.w, (row_elem0 + s * kStep) >> a.w.blocksize_log2) : 0.0f;

        floatx16_t part;
#pragma unroll
        for (int r = 0; r < 16; ++r) part[r] = 0.0f;
        const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t wv[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                // address = code byte b of the word << 8 | 4 * lane
                const uint32_t addr = __builtin_amdgcn_perm(cws[q], lane_sel, 0x0C0C0400u | ((uint32_t)(4 + b) << 8));
                wv[b] = *reinterpret_cast<const uint32_t*>(tab + addr);
            }
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
            const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, xv[q]);
            part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, part, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4 * MB; ++r) acc[r] = __builtin_fmaf(part[r], sc, acc[r]);
    }

    // reduce the S partial tiles: red[wave][r][lane] for the kept registers
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int r = 0; r < 4 * MB; ++r) red[(wave * 4 * MB + r) * 64 + lane] = acc[r];
    __syncthreads();
    // output element (i, j): register r = 4*(i/8) + i%4, lane = j + 32*((i/4)%2)
    for (int e = threadIdx.x; e < M * kRows; e += S * 64) {
        const int i = e / kRows, jj = e % kRows;
        const int r = 4 * (i / 8) + (i % 4);
        const int ln = jj + 32 * ((i / 4) % 2);
        float v = 0.0f;
        for (int w = 0; w < S; ++w) v += red[(w * 4 * MB + r) * 64 + ln];
        const int64_t nn = (int64_t)blockIdx.x * kRows + jj;
        if (nn < a.N) a.y[(int64_t)i * a.N + nn] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

// Generic path: one wave per weight row, per-element dequantization.
__global__ __launch_bounds__(256) void gemv_generic_kernel(GemvArgs a) {
    __shared__ float lev[16];
    if (threadIdx.x < 16) lev[threadIdx.x] = a.w.levels[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= a.N) return;
    const int64_t K = a.K;
    const int M = a.M;
    float acc[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
    for (int64_t k = lane; k < K; k += 64) {
        const int64_t e = n * K + k;
        const uint32_t byte = a.w.codes[e >> 1];
        const uint32_t code = (e & 1) ? (byte & 0xFu) : (byte >> 4);
        const float wq = __fmul_rn(lev[code], row_scale(a.w, e >> a.w.blocksize_log2));
        const float wd = as_float(pack_bf16x2(wq, 0.0f) << 16);   // bf16 dequantized weight
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m < M) acc[m] = __builtin_fmaf(as_float((uint32_t)a.x[(int64_t)m * K + k] << 16), wd, acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        if (m >= M) break;
        float v = acc[m];
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) a.y[(int64_t)m * a.N + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

template <int MB, int S>
hipError_t launch_mfma(const GemvArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)((a.N + kRows - 1) / kRows);
    const size_t lds = 256 * kTabCopies * sizeof(uint32_t);   // 64 KB, >= S * 4MB * 64 * 4
    hipLaunchKernelGGL((gemv_mfma_kernel<MB, S>), dim3(grid), dim3(S * 64), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const void* x, int32_t M, const MatArgs& w, void* y, hipStream_t s, const char** variant) {
    GemvArgs a;
    a.x = reinterpret_cast<const uint16_t*>(x);
    a.y = reinterpret_cast<uint16_t*>(y);
    a.w = w.w;
    a.N = w.N;
    a.K = w.K;
    a.M = M;
    const bool fast = (w.K % kStep) == 0 && (w.K % w.w.blocksize) == 0 &&
                      (reinterpret_cast<uintptr_t>(x) % 16) == 0 && (reinterpret_cast<uintptr_t>(w.w.codes) % 16) == 0;
    if (!fast) {
        *variant = "generic (per-element dequantization, one wave per row)";
        hipLaunchKernelGGL(gemv_generic_kernel, dim3((unsigned)((w.N + 3) / 4)), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const int64_t nsteps = w.K / kStep;
    *variant = "mfma 32x32x16 bf16, LDS byte-pair table, split-K over 16 waves";
    if (nsteps >= 16) return M <= 8 ? launch_mfma<1, 16>(a, s) : launch_mfma<2, 16>(a, s);
    return M <= 8 ? launch_mfma<1, 4>(a, s) : launch_mfma<2, 4>(a, s);
}

}  // namespace qk
