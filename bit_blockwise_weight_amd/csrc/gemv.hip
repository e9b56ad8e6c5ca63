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
typedef float floatx4_t __attribute__((ext_vector_type(4)));

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

// Fast path, 16 weight rows per workgroup (v_mfma_f32_16x16x32_bf16):
//   A = x (16 x 32, rows m >= M are zero), B = W^T (32 x 16 rows of the tile), so the
//   4 x 16 output registers of a wave are y[m][n] for m = 4(lane / 16) + r, n = lane % 16.
//   Lane l holds row n = l % 16 and, in 64-k block b, the 16 weights
//   k = 64 b + 16 h + [0, 16), h = l / 16 (8 code bytes, one 8-byte load); the two MFMAs
//   of a block use k = 64 b + 16 h + 8 t + [0, 8), t = 0, 1, so both stay inside one block
//   of 64 and the block scale of row n multiplies the block's partial product.
//   The S waves of a workgroup take blocks b = wave, wave + S, ... and load the codes,
//   scales and x of kBatch blocks ahead, so each wave keeps several HBM loads in flight.
constexpr int kBatch = 4;

struct GemvBatch {
    uint2 c[kBatch];      // 8 code bytes of the lane's row
    uint4 x0[kBatch];     // x[m][64 b + 16 h + 0..7]
    uint4 x1[kBatch];     // x[m][64 b + 16 h + 8..15]
    int32_t q[kBatch];    // q8 (nested) or absmax bits
    float d[kBatch];      // dq scale (nested)
};

template <int S, bool kNested>
__global__ __launch_bounds__(S * 64) void gemv16_kernel(GemvArgs a) {
    extern __shared__ uint32_t lds[];          // 64 KB pair table, reused for the reduction
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;                   // weight row of the tile (and x row m of the A operand)
    const int h = lane >> 4;                   // 16-weight group of a 64-k block
    const int64_t row = (int64_t)blockIdx.x * 16 + n;
    const bool row_ok = row < a.N;
    const int64_t rowc = row_ok ? row : a.N - 1;
    const int64_t K = a.K;
    const int64_t nblk = K / 64;
    const int64_t nbw = (nblk - wave + S - 1) / S;        // blocks of this wave
    const int M = a.M;
    const bool x_ok = n < M;
    const uint16_t* xrow = a.x + (int64_t)(x_ok ? n : 0) * K + 16 * h;
    const uint8_t* crow = a.w.codes + rowc * (K / 2) + 8 * h;
    const int64_t qb0 = (rowc * K) >> a.w.blocksize_log2;  // first quantization block of the row
    const int bshift = a.w.blocksize_log2 - 6;
    const float mean = kNested ? *a.w.dq_mean : 0.0f;

    auto load = [&](int64_t i0, GemvBatch& bt) {
#pragma unroll
        for (int p = 0; p < kBatch; ++p) {
            int64_t b = wave + (int64_t)S * (i0 + p);
            b = b < nblk ? b : nblk - 1;
            bt.c[p] = *reinterpret_cast<const uint2*>(crow + 32 * b);
            const uint4* xp = reinterpret_cast<const uint4*>(xrow + 64 * b);
            bt.x0[p] = xp[0];     // rows m >= M read row 0 and are zeroed at use
            bt.x1[p] = xp[1];
            const int64_t qb = qb0 + (b >> bshift);
            if constexpr (kNested) {
                bt.q[p] = (int32_t)a.w.q8[qb];
                bt.d[p] = a.w.dq_scale[qb / QK_DQ_BLOCK];
            } else {
                bt.q[p] = (int32_t)as_uint(a.w.absmax[qb]);
                bt.d[p] = 0.0f;
            }
        }
    };

    const uint32_t lane_sel = (uint32_t)lane * 4u;
    const char* tab = reinterpret_cast<const char*>(lds);
    floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const GemvBatch& bt, int64_t i0) {
#pragma unroll
        for (int p = 0; p < kBatch; ++p) {
            const uint32_t cws[2] = {bt.c[p].x, bt.c[p].y};
            const uint4 z = make_uint4(0, 0, 0, 0);
            const uint4 xs[2] = {x_ok ? bt.x0[p] : z, x_ok ? bt.x1[p] : z};
            floatx4_t part = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t wv[4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t addr = __builtin_amdgcn_perm(cws[t], lane_sel, 0x0C0C0400u | ((uint32_t)(4 + bb) << 8));
                    wv[bb] = *reinterpret_cast<const uint32_t*>(tab + addr);
                }
                part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xs[t]),
                                                               __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3])),
                                                               part, 0, 0, 0);
            }
            float sc;
            if constexpr (kNested) sc = __fadd_rn(__fmul_rn((float)bt.q[p], bt.d[p]), mean);
            else sc = as_float((uint32_t)bt.q[p]);
            const bool live = i0 + p < nbw;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = live ? __builtin_fmaf(part[r], sc, acc[r]) : acc[r];
        }
    };

    // two batches in flight: while one is decoded, the loads of the next are outstanding
    GemvBatch ba, bb;
    load(0, ba);
    load(kBatch, bb);
    __builtin_amdgcn_sched_barrier(0);
    {
        // pair table, 64 copies: entry i = 64 b + copy for byte b.  With 8 waves, wave w
        // writes the bytes b = w + 8 j, whose nibbles are (j / 2, w + 8 (j % 2)); the level
        // reads are uniform (scalar loads), so they do not wait for the batches in flight.
        static_assert(S == 8, "table fill assumes 8 waves");
        const int w = wave;
        const uint32_t lo0 = as_uint(a.w.levels[w]), lo1 = as_uint(a.w.levels[w + 8]);
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) {
            const float hi_nib = a.w.levels[jj >> 1];
            lds[(w + 8 * jj) * kTabCopies + lane] = pack_bf16x2(hi_nib, as_float((jj & 1) ? lo1 : lo0));
        }
    }
    __syncthreads();
    for (int64_t i0 = 0; i0 < nbw; i0 += 2 * kBatch) {
        compute(ba, i0);
        __builtin_amdgcn_sched_barrier(0);
        if (i0 + 2 * kBatch < nbw) load(i0 + 2 * kBatch, ba);
        __builtin_amdgcn_sched_barrier(0);
        compute(bb, i0 + kBatch);
        __builtin_amdgcn_sched_barrier(0);
        if (i0 + 3 * kBatch < nbw) load(i0 + 3 * kBatch, bb);
        __builtin_amdgcn_sched_barrier(0);
    }

    // reduce the S waves' tiles in a fixed order: red[wave][r][lane]
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    // output (m, nn): register r = m % 4 of lane nn + 16 (m / 4)
    for (int e = threadIdx.x; e < M * 16; e += S * 64) {
        const int m = e >> 4, nn = e & 15;
        const int r = m & 3, ln = nn + 16 * (m >> 2);
        float v = 0.0f;
        for (int w = 0; w < S; ++w) v += red[(w * 4 + r) * 64 + ln];
        const int64_t on = (int64_t)blockIdx.x * 16 + nn;
        if (on < a.N) a.y[(int64_t)m * a.N + on] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
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

template <int S, bool kNested>
hipError_t launch16(const GemvArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)((a.N + 15) / 16);
    const size_t lds = 256 * kTabCopies * sizeof(uint32_t);   // 64 KB, >= S * 4 * 64 * 4
    hipLaunchKernelGGL((gemv16_kernel<S, kNested>), dim3(grid), dim3(S * 64), lds, s, a);
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
                      (reinterpret_cast<uintptr_t>(x) % 16) == 0 && (reinterpret_cast<uintptr_t>(w.w.codes) % 8) == 0;
    if (!fast) {
        *variant = "generic (per-element dequantization, one wave per row)";
        hipLaunchKernelGGL(gemv_generic_kernel, dim3((unsigned)((w.N + 3) / 4)), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    *variant = "mfma 16x16x32 bf16, 16 rows per workgroup, LDS byte-pair table, 8 waves split-K, 4-block prefetch";
    return w.w.nested ? launch16<8, true>(a, s) : launch16<8, false>(a, s);
}

}  // namespace qk
