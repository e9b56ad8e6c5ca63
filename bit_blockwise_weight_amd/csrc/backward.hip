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
// dX: a dequantize-fused GEMM with W read untransposed (kernel notes below).  The
// LoRA term s·G comes from a pre-pass (the MFMA kernel of the forward's s·X·A, run
// on dY and B^T) and is split into bf16 hi + lo in the epilogue, times A^T.
// dA and dB are reductions over the M token rows with r outputs per column: a
// VALU kernel takes 64 C columns x one slice of rows per workgroup (fp32 FMAs in
// a fixed order) and writes per-slice partials, which a second kernel adds in
// slice order (deterministic).
#include <type_traits>

#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

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


// ---------------------------------------------------------------------------
// dX, tiled for 256 x 128 outputs per workgroup.  Wave w owns dY rows
// [64 w, 64 w + 64) and all 128 columns: 2 x 4 tiles of v_mfma_f32_32x32x16_bf16.
// The dY operand goes from global memory straight into registers: the four
// 16-deep MFMA steps of a 64-wide n step take n = n0 + 32 h + 8 kk + p for
// lane half h (the reduction order is free), so a lane's fragments for one row
// are 64 contiguous bytes.  The W^T tile (64 n x 128 k, bf16) is dequantized by
// the whole workgroup into LDS, double buffered: during step s the codes of step
// s + 1 are dequantized into the other buffer while the MFMAs of step s run, and
// the codes of steps s + 2 .. s + 4 and the dY fragments of step s + 2 are in flight.
// LDS rows of W^T are 128 bytes (64 n of one column k); the 16-byte piece c of
// column k sits in slot c ^ (((k >> 1) ^ (k >> 4)) & 7): the fragment reads of
// 16 consecutive columns are conflict-free and the dequant stores (columns 4 apart)
// are at most 2-way.  One barrier per step.
// ---------------------------------------------------------------------------
namespace dx2 {

constexpr int TM = 256;
constexpr int TN = 128;
constexpr int TK = 64;
constexpr int kXcds = 8;

__device__ __forceinline__ int wt_off(int col, int chunk) {
    return col * TK + 8 * (chunk ^ (((col >> 1) ^ (col >> 4)) & 7));
}

template <bool kLora, bool kNested>
__global__ __launch_bounds__(256) void dx_fast_kernel(DxArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t wt0[TN * TK];
    __shared__ __attribute__((aligned(16))) uint16_t wt1[TN * TK];
    // byte -> (level of the high nibble, level of the low nibble) as two fp32, 32 copies:
    // entry (b, copy) at byte offset 256 b + 8 copy, lane l reads copy l % 32 (no bank conflicts)
    __shared__ __attribute__((aligned(16))) float2 tab[256 * 32];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int fi = lane & 31, h = lane >> 5;
    const int64_t M = a.M, N = a.N, K = a.K;
    const uint32_t tiles_k = (uint32_t)((K + TN - 1) / TN);
    const uint32_t nt = (uint32_t)((M + TM - 1) / TM) * tiles_k;
    const uint32_t bid = blockIdx.x;
    // XCD x (workgroups dealt round robin) takes a contiguous run of tiles, k fastest:
    // the workgroups resident on one XCD share their dY rows through its L2.
    const uint32_t lid = (nt % kXcds == 0) ? (bid % kXcds) * (nt / kXcds) + bid / kXcds : bid;
    const int64_t m0 = (int64_t)(lid / tiles_k) * TM;
    const int64_t k0 = (int64_t)(lid % tiles_k) * TN;
    const float mu = kNested ? *a.w.dq_mean : 0.0f;
    const int64_t nsteps = N / TK;
    {
        // thread t writes copy t % 32 of the bytes b = t / 32 + 8 j: nibbles (j / 2, t / 32 + 8 (j % 2))
        const int cp = tid & 31, bg = tid >> 5;
        const float lo0 = a.w.levels[bg], lo1 = a.w.levels[bg + 8];
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) tab[(bg + 8 * jj) * 32 + cp] = make_float2(a.w.levels[jj >> 1], (jj & 1) ? lo1 : lo0);
    }

    // dY rows of this lane's fragments (rows past M read row M - 1; never stored)
    const uint16_t* yrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t row = m0 + 64 * wave + 32 * i + fi;
        row = row < M ? row : M - 1;
        yrow[i] = a.dY + row * N + 32 * h;
    }
    // W staging: rows n0 + 8 rg + i (i < 8), columns k0 + 4 kq .. + 4 (columns past K read column 0).
    // Element e = (n0 + 8 rg + i) K + k: its 2 code bytes start at e / 2 and its block is
    // e >> log2(B) = (n0 K >> log2(B)) + ((e - n0 K) >> log2(B)), n0 K being a multiple of
    // the block size (K % 64 == 0, B <= 256); the per-thread parts stay in 32 bits.
    const int rg = tid >> 5, kq = tid & 31;
    const int64_t wk = k0 + 4 * kq;
    const int64_t e0 = (int64_t)(8 * rg) * K + (wk < K ? wk : 0);
    const int lg = a.w.blocksize_log2;
    const uint32_t coff0 = (uint32_t)(e0 >> 1), halfK = (uint32_t)(K >> 1);
    uint32_t lblk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) lblk[i] = (uint32_t)((e0 + (int64_t)i * K) >> lg);
    const uint32_t copy8 = (uint32_t)(lane & 31) * 8u;
    const char* tabb = reinterpret_cast<const char*>(tab);

    uint4 y0[2][4], y1[2][4];
    // codes and scales of four steps: the loads of step s + 4 are issued in step s
    uint32_t c0[8], c1[8], c2[8], c3[8];
    float s0[8], s1[8], s2[8], s3[8];
    int32_t q0[8], q1[8], q2[8], q3[8];

    auto load_y = [&](uint4 (&y)[2][4], int64_t st) {
        st = st < nsteps ? st : nsteps - 1;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) y[i][kk] = *reinterpret_cast<const uint4*>(yrow[i] + st * TK + 8 * kk);
    };
    auto load_w = [&](uint32_t (&c)[8], float (&sv)[8], int32_t (&q)[8], int64_t st) {
        st = st < nsteps ? st : nsteps - 1;
        const uint8_t* cb = a.w.codes + st * (TK / 2) * K;
        const int64_t ub = (st * TK * K) >> lg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            c[i] = (uint32_t)*reinterpret_cast<const uint16_t*>(cb + (coff0 + (uint32_t)i * halfK));
            if constexpr (kNested) {
                q[i] = a.w.q8[ub + lblk[i]];
                sv[i] = (a.w.dq_scale + (ub >> 8))[((uint32_t)(ub & 255) + lblk[i]) >> 8];
            } else {
                sv[i] = (a.w.absmax + ub)[lblk[i]];
            }
        }
    };
    // dequantize part kk (0..3) of this thread's 8 x 4 block (column kk) -> one 16-byte LDS store;
    // the table gives the two columns of one code byte at once (parts 0, 1: byte 0; 2, 3: byte 1)
    float ascl[8];
    uint32_t cc[8];
    float2 lv[8];
    auto dequant_part = [&](uint16_t* wt, const uint32_t (&c)[8], const float (&sv)[8], const int32_t (&q)[8],
                            int kk) {
        if (kk == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // pin the use of this step's loads here: otherwise the scheduler hoists the
                // scale arithmetic of the next step above the barrier and waits for loads
                // issued a moment earlier
                uint32_t ci = c[i], qi = (uint32_t)q[i];
                float si = sv[i];
                asm volatile("" : "+v"(ci), "+v"(qi), "+v"(si));
                cc[i] = ci;
                ascl[i] = kNested ? __fadd_rn(__fmul_rn((float)(int32_t)qi, si), mu) : si;
            }
        }
        if (kk == 0 || kk == 2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t addr = __builtin_amdgcn_perm(cc[i], copy8, 0x0C0C0400u | ((uint32_t)(4 + (kk >> 1)) << 8));
                lv[i] = *reinterpret_cast<const float2*>(tabb + addr);
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float l0 = (kk & 1) ? lv[i].y : lv[i].x;
            const float l1 = (kk & 1) ? lv[i + 1].y : lv[i + 1].x;
            o[i >> 1] = pack_bf16x2(__fmul_rn(l0, ascl[i]), __fmul_rn(l1, ascl[i + 1]));
        }
        *reinterpret_cast<uint4*>(&wt[wt_off(4 * kq + kk, rg)]) = make_uint4(o[0], o[1], o[2], o[3]);
    };

    floatx16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue: dY of steps 0 and 1, W^T of step 0 in LDS, codes of step 1 in flight
    load_y(y0, 0);
    load_y(y1, 1);
    load_w(c0, s0, q0, 0);
    load_w(c1, s1, q1, 1);
    load_w(c2, s2, q2, 2);
    load_w(c3, s3, q3, 3);
    __syncthreads();                       // table
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) dequant_part(wt0, c0, s0, q0, kk);
    __builtin_amdgcn_s_waitcnt(0xC07F);    // LDS stores done (vmcnt left alone)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // one step: MFMAs of step st on (y, wt_cur); dequant of step st + 1 (cn) into wt_nxt;
    // codes of step st + 4 into cf; dY of step st + 2 into y
    auto step = [&](int64_t st, uint4 (&y)[2][4], const uint16_t* wt_cur, uint16_t* wt_nxt, uint32_t (&cn)[8],
                    float (&sn)[8], int32_t (&qn)[8], uint32_t (&cf)[8], float (&sf)[8], int32_t (&qf)[8]) {
        load_w(cf, sf, qf, st + 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8_t bfr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&wt_cur[wt_off(32 * j + fi, 4 * h + kk)]);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8_t af = __builtin_bit_cast(bf16x8_t, y[i][kk]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
            }
            dequant_part(wt_nxt, cn, sn, qn, kk);
        }
        load_y(y, st + 2);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // pairs of steps with no branch inside (a conditional second step would make the
    // compiler's wait counts at the loop head assume the loads of the skipped path)
    int64_t st = 0;
    for (; st + 3 < nsteps; st += 4) {
        step(st, y0, wt0, wt1, c1, s1, q1, c0, s0, q0);
        step(st + 1, y1, wt1, wt0, c2, s2, q2, c1, s1, q1);
        step(st + 2, y0, wt0, wt1, c3, s3, q3, c2, s2, q2);
        step(st + 3, y1, wt1, wt0, c0, s0, q0, c3, s3, q3);
    }
    if (st < nsteps) step(st, y0, wt0, wt1, c1, s1, q1, c0, s0, q0);
    if (st + 1 < nsteps) step(st + 1, y1, wt1, wt0, c2, s2, q2, c1, s1, q1);
    if (st + 2 < nsteps) step(st + 2, y0, wt0, wt1, c3, s3, q3, c2, s2, q2);

    if constexpr (kLora) {
        // + (s G) A^T: s G rows from global fp32, split into bf16 hi + lo (hi + lo = s G to 2^-16)
        const int rpad = ((a.r + 15) / 16) * 16;
        for (int kk = 0; kk < rpad; kk += 16) {
            bf16x8_t ah[2], al[2], bfr[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int64_t row = m0 + 64 * wave + 32 * i + fi;
                row = row < M ? row : M - 1;
                const float4* g = reinterpret_cast<const float4*>(a.Gs + row * rpad + kk + 8 * h);
                const float4 g0 = g[0], g1 = g[1];
                const float v[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const uint32_t hb = pack_bf16x2(v[p], 0.0f) & 0xFFFFu;
                    ah[i][p] = __builtin_bit_cast(__bf16, (uint16_t)hb);
                    al[i][p] = (__bf16)(v[p] - as_float(hb << 16));
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int64_t col = k0 + 32 * j + fi;
                col = col < K ? col : K - 1;
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int jj = kk + 8 * h + p;
                    bfr[j][p] = __builtin_bit_cast(__bf16, jj < a.r ? a.A[col * a.r + jj] : (uint16_t)0);
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bfr[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bfr[j], acc[i][j], 0, 0, 0);
                }
        }
    }

    // lane holds C[8 b + 4 h + q][fi] in register 4 b + q
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t gk = k0 + 32 * j + fi;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gm = m0 + 64 * wave + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
                if (gm < M && gk < K) a.dX[gm * K + gk] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
            }
        }
    }
}

}  // namespace dx2

// Partial reductions over a slice of the M rows: part[slice][l][j] = sum over the
// rows m of the slice of P[m][l] * Q[m][j] (P bf16 [M, L], Q fp32 [M, rpad]).
// A workgroup takes 64 C columns (C per lane, C rpad <= 64 accumulators) and one
// slice; its 4 waves take the rows m = r0 + w, r0 + w + 4, ... in increasing
// order, with the Q row read through the scalar cache (it is the same for the whole
// wave), and the 4 wave sums are added in wave order through LDS.
template <int R16, int C>
__global__ __launch_bounds__(256) void tn_partial_kernel(const uint16_t* __restrict__ P, int64_t L,
                                                         const float* __restrict__ Q, int64_t M,
                                                         float* __restrict__ part) {
    constexpr int kRp = 16 * R16;
    constexpr int kAcc = C * kRp;
    __shared__ float red[3 * kAcc * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t l0 = ((int64_t)blockIdx.x * 64 + lane) * C;
    const bool ok = l0 < L;                  // L % C == 0: a lane's C columns are all in range or all out
    const uint16_t* pcol = P + (ok ? l0 : 0);
    const int slice = blockIdx.y;
    const int64_t r0 = M * slice / kSlices, r1 = M * (slice + 1) / kSlices;
    float acc[kAcc];
#pragma unroll
    for (int x = 0; x < kAcc; ++x) acc[x] = 0.0f;
#pragma unroll 4
    for (int64_t m = r0 + wave; m < r1; m += 4) {
        float p[C];
        if constexpr (C == 4) {
            const uint2 v = *reinterpret_cast<const uint2*>(pcol + m * L);
            p[0] = bf16_lo(v.x); p[1] = bf16_hi(v.x); p[2] = bf16_lo(v.y); p[3] = bf16_hi(v.y);
        } else if constexpr (C == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(pcol + m * L);
            p[0] = bf16_lo(v); p[1] = bf16_hi(v);
        } else {
            p[0] = as_float((uint32_t)pcol[m * L] << 16);
        }
        const float* q = Q + m * kRp;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int j = 0; j < kRp; ++j) acc[c * kRp + j] = __builtin_fmaf(p[c], q[j], acc[c * kRp + j]);
    }
    if (wave > 0) {
#pragma unroll
        for (int x = 0; x < kAcc; ++x) red[((wave - 1) * kAcc + x) * 64 + lane] = acc[x];
    }
    __syncthreads();
    if (wave == 0 && ok) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int x = 0; x < kAcc; ++x) acc[x] += red[(w * kAcc + x) * 64 + lane];
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int j = 0; j < kRp; ++j) part[((int64_t)slice * L + l0 + c) * kRp + j] = acc[c * kRp + j];
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
    const int C = r16 == 1 ? 4 : (r16 == 2 ? 2 : 1);     // L is a multiple of 64
    const dim3 grid((unsigned)((L / C + 63) / 64), kSlices);
    switch (r16) {
        case 1: hipLaunchKernelGGL((tn_partial_kernel<1, 4>), grid, dim3(256), 0, s, P, L, Q, M, part); break;
        case 2: hipLaunchKernelGGL((tn_partial_kernel<2, 2>), grid, dim3(256), 0, s, P, L, Q, M, part); break;
        case 3: hipLaunchKernelGGL((tn_partial_kernel<3, 1>), grid, dim3(256), 0, s, P, L, Q, M, part); break;
        default: hipLaunchKernelGGL((tn_partial_kernel<4, 1>), grid, dim3(256), 0, s, P, L, Q, M, part); break;
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
    const int64_t nt = ((M + dx2::TM - 1) / dx2::TM) * ((K + dx2::TN - 1) / dx2::TN);
    if (nt > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nt);
    if (lora) {
        if (w.w.nested) hipLaunchKernelGGL((dx2::dx_fast_kernel<true, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((dx2::dx_fast_kernel<true, false>), grid, dim3(256), 0, s, a);
    } else {
        if (w.w.nested) hipLaunchKernelGGL((dx2::dx_fast_kernel<false, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((dx2::dx_fast_kernel<false, false>), grid, dim3(256), 0, s, a);
    }
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
