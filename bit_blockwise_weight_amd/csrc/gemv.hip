// Decode-time GEMV with the dequantized weight, for gfx950:
//     y[m, n] = sum_k x[m, k] * deq(W)[n, k],   m < M <= 16
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 【代码】 (the 4-bit linear
// layer's forward is dequantize + matmul); "Tim Dettmers 如何用 bitsandbytes 與
// QLoRA 降低 LLM 訓練門檻？", section on speed (unpacking and dequantizing must be
// fused, or 4-bit can be slower than 16-bit).  The weight is never written out.
//
// Fast path (K a multiple of 64 and of the block size, 16-byte aligned codes and x):
//   * A workgroup owns 16 weight rows; its S waves split K in chunks of 512
//     (wave w takes chunks w, w + S, ...).  S = 4 (80 KB of LDS: two workgroups
//     per CU, one loading while the other computes) when there are at least two
//     tiles per CU and K <= 4096; S = 8 otherwise.
//   * Codes are loaded so that one instruction fetches 256 contiguous bytes from
//     each of 4 rows; each wave writes its chunk to its own LDS area (no barrier)
//     and reads it back in MFMA layout.  In that area the 16-byte piece p of row r
//     sits in slot 16 r + (p ^ r), so the 16 rows a fragment read touches fall in
//     16 different bank groups.  The next chunk's codes, x and scales are loaded
//     before the current chunk is computed, by loads outside any branch.
//   * v_mfma_f32_16x16x32_bf16 with A = x (16 x 32, rows m >= M are zero) and
//     B = W^T (32 x 16 rows), so the 4 output registers of lane l are y[m][n] for
//     m = 4(l / 16) + r, n = l % 16.  Lane l holds row n = l % 16 and, in 64-k block
//     b, the 16 weights k = 64 b + 16 h + [0, 16), h = l / 16; the block's two MFMAs
//     take k = 64 b + 16 h + 8 t + [0, 8), t = 0, 1, so both stay inside one block of
//     64 and the row's block scale a' (fp32) multiplies the block's partial product:
//     one FMA per output register per block, none per weight.
//   * Decoding: an LDS table maps a code byte to the pair (bf16 level of the high
//     nibble, bf16 level of the low nibble) as one dword, replicated 64 times and
//     interleaved so that lane l reads copy l: the address (byte << 8 | 4l) is one
//     v_perm, the read never conflicts.
//   * The S waves' partial tiles are summed through LDS in a fixed order.
// The levels are used as bf16 and the block scale is applied in fp32 after the
// bf16 products; the result agrees with the fp64 product on the bf16-dequantized
// weight within the documented tolerance.
//
// Generic path (any K, blocks straddling rows): one wave per row, each lane walks
// k = lane, lane + 64, ... and dequantizes each weight exactly as the dequantize
// kernel does (bf16 of level * a'), with fp32 accumulation.
#include <type_traits>

#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

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

// Fast path kernel (see the top of the file).
constexpr int kChunkK = 512;                   // k per chunk (8 blocks of 64)
constexpr int kChunkBlocks = kChunkK / 64;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct ChunkRegs {
    u32x4_t c[4];                // 16-byte code pieces of this lane (4 rows x 256 bytes per wave load)
    uint4 x[kChunkBlocks][2];    // x[m][c0 + 64 b + 16 h + 8 t .. +8], t = 0, 1
    int32_t q[kChunkBlocks];     // q8 (nested) or absmax bits
    float d[kChunkBlocks];       // dq scale (nested)
};

template <bool kNested, int S>
__global__ __launch_bounds__(S * 64) void gemv_lds_kernel(GemvArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t tab[256 * kTabCopies];   // 64 KB byte -> bf16 pair
    __shared__ __attribute__((aligned(1024))) uint4 cb[S][256];               // codes chunk, 4 KB per wave
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;                   // weight row of the tile (and x row m of the A operand)
    const int h = lane >> 4;                   // 16-weight group of a 64-k block
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t K = a.K;
    const int64_t nblk = K / 64;
    const int64_t nchunk = (K + kChunkK - 1) / kChunkK;
    const int64_t ncw = (nchunk - wave + S - 1) / S;       // chunks of this wave
    const int M = a.M;
    const bool x_ok = n < M;
    const uint16_t* xrow = a.x + (int64_t)(x_ok ? n : 0) * K + 16 * h;
    const int64_t rowc = n0 + n < a.N ? n0 + n : a.N - 1;
    const int64_t qb0 = (rowc * K) >> a.w.blocksize_log2;  // first quantization block of the row
    const int bshift = a.w.blocksize_log2 - 6;
    const float mean = kNested ? *a.w.dq_mean : 0.0f;
    const int64_t row_bytes = K / 2;

    // code loads: load i, lane L fetches piece (L % 16) ^ r of row r = 4 i + L / 16
    const uint8_t* csrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int64_t gr = n0 + r < a.N ? n0 + r : a.N - 1;
        csrc[i] = a.w.codes + gr * row_bytes + 16 * ((lane & 15) ^ r);
    }
    auto load = [&](int64_t c, ChunkRegs& cr) {
        const int64_t cc = c < nchunk ? c : nchunk - 1;
        const int64_t cbase = cc * (kChunkK / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // pieces past the end of a row (last, partial chunk) are clamped and never used
            const int64_t off = cbase + 16 * ((lane & 15) ^ (4 * i + (lane >> 4)));
            const int64_t adj = off + 16 <= row_bytes ? 0 : row_bytes - 16 - off;
            cr.c[i] = *reinterpret_cast<const u32x4_t*>(csrc[i] + cbase + adj);
        }
#pragma unroll
        for (int b = 0; b < kChunkBlocks; ++b) {
            int64_t blk = cc * kChunkBlocks + b;
            blk = blk < nblk ? blk : nblk - 1;
            const uint4* xp = reinterpret_cast<const uint4*>(xrow + 64 * blk);
            cr.x[b][0] = xp[0];     // rows m >= M read row 0 and are zeroed at use
            cr.x[b][1] = xp[1];
            const int64_t qb = qb0 + (blk >> bshift);
            if constexpr (kNested) {
                cr.q[b] = (int32_t)a.w.q8[qb];
                cr.d[b] = a.w.dq_scale[qb / QK_DQ_BLOCK];
            } else {
                cr.q[b] = (int32_t)as_uint(a.w.absmax[qb]);
                cr.d[b] = 0.0f;
            }
        }
    };
    u32x4_t* mine = reinterpret_cast<u32x4_t*>(cb[wave]);
    auto stage = [&](const ChunkRegs& cr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[i * 64 + lane] = cr.c[i];    // slot 64 i + L = 16 r + (piece ^ r)
    };

    floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t lane_sel = (uint32_t)lane * 4u;
    const char* tabb = reinterpret_cast<const char*>(tab);
    const char* mb = reinterpret_cast<const char*>(mine);
    auto compute = [&](int64_t c, const ChunkRegs& cr) {
#pragma unroll
        for (int b = 0; b < kChunkBlocks; ++b) {
            const int piece = 2 * b + (h >> 1);
            const uint2 cw = *reinterpret_cast<const uint2*>(mb + (16 * n + (piece ^ n)) * 16 + 8 * (h & 1));
            const uint32_t cws[2] = {cw.x, cw.y};
            floatx4_t part = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t wv[4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint32_t addr = __builtin_amdgcn_perm(cws[t], lane_sel, 0x0C0C0400u | ((uint32_t)(4 + bb) << 8));
                    wv[bb] = *reinterpret_cast<const uint32_t*>(tabb + addr);
                }
                const uint4 z = make_uint4(0, 0, 0, 0);
                part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x_ok ? cr.x[b][t] : z),
                                                               __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3])),
                                                               part, 0, 0, 0);
            }
            float sc;
            if constexpr (kNested) sc = __fadd_rn(__fmul_rn((float)cr.q[b], cr.d[b]), mean);
            else sc = as_float((uint32_t)cr.q[b]);
            const bool live = c * kChunkBlocks + b < nblk;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = live ? __builtin_fmaf(part[r], sc, acc[r]) : acc[r];
        }
    };

    const int64_t c0 = wave;
    ChunkRegs ra, rb;
    load(c0, ra);   // clamped: a wave without chunks reads a valid one and never uses it
    {
        // pair table, 64 copies: entry i = 64 b + copy for byte b.  Wave w writes the bytes
        // b = w + S j, whose nibbles are (j / (16 / S), w + S (j % (16 / S))); the level reads
        // are uniform (scalar loads), so they do not wait for the loads in flight.
        constexpr int kLo = 16 / S;
        float lo[kLo];
#pragma unroll
        for (int q = 0; q < kLo; ++q) lo[q] = a.w.levels[wave + S * q];
#pragma unroll
        for (int jj = 0; jj < 256 / S; ++jj) {
            const float hi_nib = a.w.levels[jj / kLo];
            tab[(wave + S * jj) * kTabCopies + lane] = pack_bf16x2(hi_nib, lo[jj % kLo]);
        }
    }
    // a bare barrier: __syncthreads() would add a fence that waits for the loads in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) (the table writes), vmcnt and expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    stage(ra);
    // Two chunks per iteration, the register sets alternating by name (a copy would wait
    // for its loads): load the next chunk, compute this one from LDS, then stage the next.
    // Every load inside the loop is unconditional and the last one or two chunks are
    // peeled: a load under a branch merges the wait counts at the join, and the compute
    // of this chunk would then wait for the next chunk's loads.
    int64_t i = 0;
    for (; i + 2 < ncw; i += 2) {
        const int64_t c = c0 + (int64_t)S * i;
        load(c + S, rb);
        compute(c, ra);
        stage(rb);
        load(c + 2 * S, ra);
        compute(c + S, rb);
        stage(ra);
    }
    if (ncw - i == 2) {
        const int64_t c = c0 + (int64_t)S * i;
        load(c + S, rb);
        compute(c, ra);
        stage(rb);
        compute(c + S, rb);
    } else if (ncw - i == 1) {
        compute(c0 + (int64_t)S * i, ra);
    }

    // reduce the S waves' tiles in a fixed order: red[wave][r][lane] (over the table)
    __syncthreads();
    float* red = reinterpret_cast<float*>(tab);
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    // output (m, nn): register r = m % 4 of lane nn + 16 (m / 4)
    for (int e = threadIdx.x; e < M * 16; e += S * 64) {
        const int m = e >> 4, nn = e & 15;
        const int r = m & 3, ln = nn + 16 * (m >> 2);
        float v = 0.0f;
        for (int w = 0; w < S; ++w) v += red[(w * 4 + r) * 64 + ln];
        const int64_t on = n0 + nn;
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
    *variant = "mfma 16x16x32 bf16, 16 rows per workgroup, codes staged through LDS in 512-k chunks, 4 or 8 waves split-K";
    const unsigned grid = (unsigned)((a.N + 15) / 16);
    // 4 waves (80 KB of LDS, two workgroups per CU, so one's loads overlap the other's
    // compute) when there are at least two tiles per CU and K fits 8 chunks; 8 waves
    // (one workgroup per CU, more loads in flight per tile) otherwise
    const bool four = grid >= 2u * (unsigned)device_cu_count() && w.K <= 8 * kChunkK;
    if (four) {
        if (w.w.nested) hipLaunchKernelGGL((gemv_lds_kernel<true, 4>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((gemv_lds_kernel<false, 4>), dim3(grid), dim3(256), 0, s, a);
    } else {
        if (w.w.nested) hipLaunchKernelGGL((gemv_lds_kernel<true, 8>), dim3(grid), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((gemv_lds_kernel<false, 8>), dim3(grid), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace qk
