// Decode-time GEMV with the dequantized weight, for gfx950:
//     y[m, n] = sum_k x[m, k] * deq(W)[n, k],   m < M <= 16
// "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 【代码】 (the 4-bit linear
// layer's forward is dequantize + matmul); "Tim Dettmers 如何用 bitsandbytes 與
// QLoRA 降低 LLM 訓練門檻？", section on speed (unpacking and dequantizing must be
// fused, or 4-bit can be slower than 16-bit).  The weight is never written out.
//
// Fast path (every row length a multiple of 64 and of the block size, 16-byte
// aligned codes and x), one launch for a whole group of weights (a layer: up to 16
// slices of weights that share nothing but the launch, more launches beyond), the
// weights cut into tiles of 16 rows sorted by row length:
//   * M = 1: gemv_group_kernel.  One 8-wave workgroup per CU walks the tiles wg,
//     wg + G, ...; in a tile, wave w takes the 512-k jobs w, w + 8, ... and keeps
//     its partial 16 outputs in LDS until the end, when the 8 partials of every
//     tile are added in wave order (no barrier inside the loop).
//   * 2 <= M <= 16: gemv_rows_kernel.  One workgroup per group of 8 consecutive
//     tiles of one slice; each wave owns a tile and walks its rows from k = 0 to K,
//     the 8 waves taking the same job at the same time so that the x chunk of a
//     job (M rows x 1 KB) is copied to LDS once and shared.  At M <= 4 two waves
//     share a tile (its even and its odd jobs) and a workgroup owns 4 tiles.
//   Both: a job's codes (16 rows x 256 bytes) arrive by 4 buffer loads with the
//   LDS bit and the nontemporal hint, each fetching 256 contiguous bytes of 4 rows
//   into the wave's own LDS slot (piece p of row r in slot 16 r + (p ^ r), so the
//   16 rows a fragment read touches fall in 16 different bank groups); the scales
//   come by one or two plain loads, x by LDS copies as well.  Two slots per wave:
//   the next job's loads are issued before the current job's compute, and explicit
//   s_waitcnt counts (the compiler's own waits drained every copy in flight)
//   let a job wait for its own loads only.
//   * v_mfma_f32_16x16x32_bf16 with A = x (16 x 32; A rows m >= M repeat row M - 1
//     and feed outputs that are never stored) and B = W^T (32 x 16 rows), so the 4
//     output registers of lane l are y[m][n] for m = 4(l / 16) + r, n = l % 16.
//     Lane l holds row n = l % 16 and, in 64-k block b, the 16 weights k = 64 b +
//     16 h + [0, 16), h = l / 16; the block's two MFMAs take k = 64 b + 16 h + 8 t
//     + [0, 8), t = 0, 1, so both stay inside one block of 64 and the row's block
//     scale a' (fp32) multiplies the block's partial product: one FMA per output
//     register per block, none per weight.
//   * Decoding: an LDS table maps a code byte to the pair (bf16 level of the high
//     nibble, bf16 level of the low nibble) as one dword, replicated 64 times and
//     interleaved so that lane l reads copy l: the address (byte << 8 | 4l) is one
//     v_perm, the read never conflicts.
// The levels are used as bf16 and the block scale is applied in fp32 after the
// bf16 products; the result agrees with the fp64 product on the bf16-dequantized
// weight within the documented tolerance.
//
// Generic path (any K, blocks straddling rows): one wave per row, each lane walks
// k = lane, lane + 64, ... and dequantizes each weight exactly as the dequantize
// kernel does (bf16 of level * a'), with fp32 accumulation.
#include <algorithm>
#include <cstring>
#include <type_traits>
#include <vector>

#include "qk_internal.h"
#include "qk_device.h"

namespace qk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kStep = 64;          // k per step
constexpr int kTabCopies = 64;
// cache policy of the code loads: nontemporal (each code byte is read once; a stream of
// nontemporal 16-byte loads reads 6.4 TB/s against 6.0 for plain loads).  The block
// scales keep the default policy: a job reads 8 bytes of a row's 128-byte line and the
// next job of the tile the next 8, from L2.
constexpr int kStream = 2;
// parts of a job's loads (the K-split kernel issues its codes and its x at different times)
constexpr int kLoadCodes = 1;   // block scales and codes
constexpr int kLoadX = 2;       // x rows
// rows of x from which the row-split kernel (shared x chunk) replaces the K-split one
constexpr int kRowsMinM = 2;

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
// A slice of rows of one weight (a whole weight unless it is very tall).
struct GemvTask {
    const uint16_t* x;       // [M, K] bf16 bits
    uint16_t* y;             // y of the slice's first row: y[m * ystride + row]
    const uint8_t* codes;    // codes of the slice's first row
    const void* sc;          // the weight's q8 (int8, nested) or absmax (fp32), from its first block
    const float* dq_scale;   // nested
    const float* dq_mean;    // nested
    int64_t N;               // rows of the slice
    int64_t ystride;         // rows of the weight
    int64_t qbase;           // quantization block of the slice's first element
    int32_t K;
    int32_t nchunk;          // ceil(K / 512)
    int32_t jobs;            // jobs per wave per tile: ceil(nchunk / S)
    int32_t item0;           // first tile of the slice in the launch
    int32_t code_bytes;      // N * K / 2 of the slice (< 2^31)
    int32_t sc_bytes;        // bytes of the weight's q8 (rounded up to dwords) or absmax (< 2^31)
    int32_t dq_bytes;        // bytes of the weight's dq_scale (nested)
    int32_t pad;
};

struct GemvGroup {
    GemvTask t[kMaxGemvTasks];
    float levels[16];
    int32_t ntasks;
    int32_t nitems;          // tiles of 16 rows over all slices (<= out_slots * grid)
    int32_t M;
    int32_t qs;              // log2(block size) - 6
};

constexpr int kChunkK = 512;                   // k per job (8 blocks of 64)
constexpr int kChunkBlocks = kChunkK / 64;
// tiles per workgroup whose partial sums LDS holds until the end of the kernel
__host__ __device__ constexpr int out_slots(int S, int MX) { return S * MX <= 8 ? 32 : 16; }
// 16-byte units per staged x row (64 used, the rest pads the rotation of rows m > 0)
__host__ __device__ constexpr int x_pitch(int MX) { return MX == 1 ? 64 : 80; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// Rotation of staged x row m: unit u of the row sits in slot m * kXPitch + u + xrot(m).  A
// fragment read of one (block, half) touches unit 8 b + 2 h + t of rows m < M in lanes
// (h, m); with this rotation those 16-byte reads of rows 0..3 fall in 16 distinct groups
// of 4 banks, and the writes of one row (unit = lane) are consecutive.
__device__ __forceinline__ int xrot(int m) { return 8 * (m & 1) + (m >> 1); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One job's registers: the scale inputs (the codes and x rows of a job go to LDS directly).
struct JobRegs {
    u32x3_t q;                   // nested: q8 bytes of the job (aligned: the first 8; else 12 from qf & ~3)
    u32x4_t f0, f1;              // plain: absmax of the job's quantization blocks (up to 8)
    u32x2_t d;                   // nested: dq scale of the job (aligned), or of its first dq block and the next
    uint32_t qinfo;              // nested, not aligned: (qf & 3) | (blocks left in the first dq block) << 2
};

// S waves per workgroup, MX rows of x staged per job (M <= MX), C copies of the code table,
// QS = log2(block size) - 6 (a job's 8 blocks of 64 fall in 8 >> QS quantization blocks),
// kAligned: every row length of the launch is a multiple of 512, so a job's quantization
// blocks are one aligned run inside one double-quantization block.
//
// A job is 16 rows x 512 k: its codes (4 KB) and x rows (M x 1 KB) are copied from memory
// straight into one of the wave's two LDS slots by buffer loads with the LDS bit, 16 bytes
// per lane and instruction (so 4 + M vector memory instructions carry a job's bulk, with no
// registers and no LDS writes of the wave's own); the scales come with two more.  The two
// slots are separate LDS objects, so the wait before reading one leaves the other's copies
// in flight.  The lane offsets of a tile's rows are computed once per tile; the job's chunk
// enters the loads as their scalar offset where the chunk cannot run past the row.
template <int S, int MX, int C, bool kNested, int QS, bool kAligned>
__global__ __launch_bounds__(S * 64, 1) void gemv_group_kernel(GemvGroup g) {
    constexpr int kR = MX < 4 ? MX : 4;        // output registers of a lane that can hold a row m < M
    constexpr int kXPitch = x_pitch(MX);
    constexpr int kSlotX = MX * kXPitch;       // 16-byte units of a staged x slot
    constexpr int kSlots = out_slots(S, MX);
    constexpr int kJobQ = kChunkBlocks >> QS;  // quantization blocks per job
    // vector memory instructions per job: the scales (two, or one absmax load when a job
    // has at most 4 blocks), the 4 code copies and the MX x copies
    constexpr int kLoads = (kNested || QS == 0 ? 2 : 1) + 4 + MX;
    // byte -> bf16 pair, C copies; the highest alignment puts it at LDS offset 0, so the
    // table base fits the read instructions' immediate offset (no add per lookup)
    __shared__ __attribute__((aligned(4096))) uint32_t tab[256 * C];
    __shared__ __attribute__((aligned(1024))) uint4 cb0[S * 256];             // codes, slot 0 (4 KB per wave)
    __shared__ __attribute__((aligned(1024))) uint4 cb1[S * 256];             // codes, slot 1
    __shared__ __attribute__((aligned(16))) uint4 xs0[S * kSlotX];            // x rows, slot 0
    __shared__ __attribute__((aligned(16))) uint4 xs1[S * kSlotX];            // x rows, slot 1
    __shared__ __attribute__((aligned(16))) float part[kSlots][S][kR][16];    // each wave's partial tiles
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;                   // weight row of the tile (and x row m of the A operand)
    const int h = lane >> 4;                   // 16-weight group of a 64-k block
    const int M = g.M;
    const int32_t G = (int32_t)gridDim.x;
    const int32_t wg = (int32_t)blockIdx.x;

    // This workgroup takes the tiles wg, wg + G, ...; in each, wave w takes the jobs
    // (chunks of 512 k) w, w + S, ...  Every wave of the workgroup sees the same tiles and
    // job counts.  The load cursor holds its slice's buffers and, for its tile, this lane's
    // offsets of the code rows and of its row's first scale; the compute cursor only needs
    // the job count and the mean (a scalar load when it changes slice).
    struct LoadCur {
        int32_t item, task, j, jobs, nchunk, K, item0, code_bytes, sc_bytes, dq_bytes;
        const void* codes;
        const void* x;
        const void* sc;
        const void* dq_scale;
        uint32_t crow[4];          // code offset of tile row 4 i + lane / 16 and this lane's piece (per slice)
        uint32_t qrow;             // scale index of tile row n's first block, from the tile's first (per slice)
        uint32_t qbase;            // scale index of the slice's first block
        uint32_t tcode;            // code offset of the tile's first row (per tile, uniform)
        uint32_t tq;               // scale index of the tile's first block (per tile, uniform)
    };
    struct CompCur {
        int32_t item, task, j, jobs;
        float mu;
    };
    auto task_from = [&](int32_t item, int32_t t) {
        while (t + 1 < g.ntasks && item >= g.t[t + 1].item0) ++t;
        return t;
    };
    auto set_load_task = [&](LoadCur& c, int32_t t) {
        const GemvTask& T = g.t[t];
        c.task = t;
        c.jobs = T.jobs;
        c.nchunk = T.nchunk;
        c.K = T.K;
        c.item0 = T.item0;
        c.code_bytes = T.code_bytes;
        c.sc_bytes = T.sc_bytes;
        c.dq_bytes = T.dq_bytes;
        c.codes = T.codes;
        c.x = T.x;
        c.sc = T.sc;
        c.dq_scale = T.dq_scale;
        // lane offsets relative to a tile's first row: they change only with the slice
        const uint32_t row_bytes = (uint32_t)(T.K / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + (lane >> 4);
            c.crow[i] = (uint32_t)r * row_bytes + 16u * (uint32_t)((lane & 15) ^ r);
        }
        c.qrow = (uint32_t)n * (uint32_t)(T.K >> (QS + 6));
        c.qbase = (uint32_t)T.qbase;
    };
    // the tile's first row enters the loads' scalar offsets; rows past the slice's end
    // then lie past the code buffer's range and read zero (their outputs are never
    // stored), and their scales are other rows' or zero.  On gfx950 the range check of
    // a raw buffer load compares the vector plus the scalar offset with the buffer's
    // size (measured: with 512 bytes in range and a scalar offset of 256, lanes whose
    // vector offset is 256 or more read zero although their addresses lie inside the
    // allocation), so a scalar offset cannot carry a load past the buffer.
    auto enter_tile = [&](LoadCur& c) {
        const uint32_t n0 = (uint32_t)(c.item - c.item0) * 16u;
        c.tcode = n0 * (uint32_t)(c.K / 2);
        c.tq = c.qbase + n0 * (uint32_t)(c.K >> (QS + 6));
    };
    auto set_comp_task = [&](CompCur& c, int32_t t) {
        c.task = t;
        c.jobs = g.t[t].jobs;
        // a scalar load (constant address space: the mean does not change during the
        // kernel): no vector memory operation under the task-switch condition
        c.mu = kNested ? *(const __attribute__((address_space(4))) float*)(uintptr_t)g.t[t].dq_mean : 0.0f;
    };
    auto advance_load = [&](LoadCur& c) {
        if (++c.j == c.jobs) {
            c.j = 0;
            c.item += G;
            if (c.item < g.nitems) {
                if (c.task + 1 < g.ntasks && c.item >= g.t[c.task + 1].item0)
                    set_load_task(c, task_from(c.item, c.task + 1));
                enter_tile(c);
            }
        }
    };
    auto advance_comp = [&](CompCur& c) {
        if (++c.j == c.jobs) {
            c.j = 0;
            c.item += G;
            if (c.item < g.nitems && c.task + 1 < g.ntasks && c.item >= g.t[c.task + 1].item0)
                set_comp_task(c, task_from(c.item, c.task + 1));
        }
    };
    LoadCur lc;
    lc.item = wg;
    lc.j = 0;
    set_load_task(lc, task_from(wg, 0));
    enter_tile(lc);
    CompCur cc;
    cc.item = wg;
    cc.j = 0;
    set_comp_task(cc, lc.task);

    // what = kLoadCodes (scales and codes), kLoadX (x rows) or both
    auto load = [&](const LoadCur& c, JobRegs& jr, auto slot, auto what) {
        constexpr bool kB = decltype(slot)::value;
        constexpr int kWhat = decltype(what)::value;
        // a job past the end of the work (after the last one) reloads its last tile's rows
        // (valid memory, mostly from the cache); it is never stored
        const __amdgpu_buffer_rsrc_t lcr = buf_rsrc(c.codes, c.code_bytes);
        const __amdgpu_buffer_rsrc_t lxr = buf_rsrc(c.x, M * c.K * 2);
        const __amdgpu_buffer_rsrc_t lsr = buf_rsrc(c.sc, c.sc_bytes);
        const __amdgpu_buffer_rsrc_t ldr = buf_rsrc(c.dq_scale, c.dq_bytes);
        // (the builtins below take plainly typed locals: a member of the cursor, whose type
        // depends on the template, makes host compilation drop the kernel's launch stub)
        const int32_t K = c.K;
        const uint32_t qrow = c.qrow;
        const uint32_t tcode = c.tcode;
        const uint32_t tq = c.tq;
        const uint32_t crow[4] = {c.crow[0], c.crow[1], c.crow[2], c.crow[3]};
        const int32_t ch = c.j * S + wave;
        const bool live = ch < c.nchunk;                 // an idle wave's chunk: x reads zero
        const int32_t chc = live ? ch : c.nchunk - 1;
        // the job's quantization blocks of row n are consecutive from qf on
        const uint32_t qs0 = tq + (uint32_t)(chc * kJobQ);   // uniform part of the scale index
        const uint32_t qf = qrow + qs0;
        if constexpr ((kWhat & kLoadCodes) != 0) {
            if constexpr (kNested) {
                if constexpr (kAligned) {
                    // the job's kJobQ q8 bytes start at a multiple of kJobQ (8, 4 or 2)
                    if constexpr (QS == 0)
                        jr.q.xy = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(lsr, qrow, qs0, 0));
                    else
                        jr.q.x = __builtin_amdgcn_raw_buffer_load_b32(lsr, qf & ~3u, 0, 0);
                    if constexpr (QS == 2) jr.qinfo = qf & 3u;
                    jr.d.x = __builtin_amdgcn_raw_buffer_load_b32(ldr, (qf / QK_DQ_BLOCK) * 4u, 0, 0);
                } else {
                    jr.q = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(lsr, qf & ~3u, 0, 0));
                    jr.d = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(ldr, (qf / QK_DQ_BLOCK) * 4u, 0, 0));
                    jr.qinfo = (qf & 3u) | ((QK_DQ_BLOCK - qf % QK_DQ_BLOCK) << 2);
                }
            } else {
                if constexpr (kAligned) {
                    jr.f0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lsr, qrow * 4u, qs0 * 4u, 0));
                    if constexpr (QS == 0)
                        jr.f1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lsr, qrow * 4u, qs0 * 4u + 16u, 0));
                } else {
                    jr.f0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lsr, qf * 4u, 0, 0));
                    if constexpr (QS == 0)
                        jr.f1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lsr, qf * 4u + 16u, 0, 0));
                }
            }
            __attribute__((address_space(3))) char* cdst =
                (__attribute__((address_space(3))) char*)reinterpret_cast<char*>(kB ? cb1 : cb0) + wave * 4096;
            // codes: load i, lane L fetches piece (L % 16) ^ r of row r = 4 i + L / 16, which lands
            // in slot unit 64 i + L
            if constexpr (kAligned) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(lcr, (lds_ptr_t)(cdst + i * 1024), 16, crow[i],
                                                             tcode + (uint32_t)chc * (kChunkK / 2), 0, kStream);
            } else {
                // pieces past the end of a row, in a partial chunk, are clamped to the row's last
                // 16 bytes (their x is zero); the offset stays in the range-checked vector part
                const uint32_t row_bytes = (uint32_t)(K / 2);
                const uint32_t cofs = (uint32_t)chc * (kChunkK / 2);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * i + (lane >> 4);
                    const uint32_t piece = 16u * (uint32_t)((lane & 15) ^ r);
                    const uint32_t within = cofs + piece + 16u <= row_bytes ? cofs : row_bytes - 16u - piece;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(lcr, (lds_ptr_t)(cdst + i * 1024), 16, crow[i] + within,
                                                             tcode, 0, kStream);
                }
            }
        }
        if constexpr ((kWhat & kLoadX) == 0) return;
        // x rows m < MX of the job's k, 16 bytes per lane: unit L of row m lands in slot unit
        // m * kXPitch + xrot(m) + L.  An idle wave's chunk and the k past the row in a partial
        // chunk take an offset beyond the buffer and read zero, so those products vanish
        // whatever codes and scales the job holds; rows past M are never stored.
        __attribute__((address_space(3))) char* xdst =
            (__attribute__((address_space(3))) char*)reinterpret_cast<char*>(kB ? xs1 : xs0) + wave * (kSlotX * 16);
        const bool xin = live && ch * kChunkK + 8 * lane < K;
        const uint32_t xo = xin ? (uint32_t)(ch * (kChunkK * 2) + 16 * lane) : 0x80000000u;
#pragma unroll
        for (int m = 0; m < MX; ++m)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lxr, (lds_ptr_t)(xdst + (m * kXPitch + xrot(m)) * 16), 16,
                                                     xo, (uint32_t)(m * K * 2), 0, 0);
    };

    floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t lane_sel = C == 64 ? (uint32_t)lane * 4u : (uint32_t)(lane & 31) * 8u;
    const char* tabb = reinterpret_cast<const char*>(tab);
    // A operand rows m >= M are another row's data: they only feed output rows that are
    // never stored
    const int xrow = n < M ? n : M - 1;
    const int xunit = xrow * kXPitch + xrot(xrow) + 2 * h;
    // A job: its scales are taken from the registers and its code words from the LDS slot
    // first; once those reads have returned, refill() issues the scale and code loads of the
    // job two ahead into the same registers and slot, so they are in flight while this job's
    // table lookups and MFMAs run (x stays in its slot until the end of the job).
    auto compute = [&](const CompCur& c, const JobRegs jr, auto slot, auto&& refill) {
        constexpr bool kB = decltype(slot)::value;
        const char* mb = reinterpret_cast<const char*>(kB ? cb1 : cb0) + wave * 4096;
        const u32x4_t* xf = reinterpret_cast<const u32x4_t*>(kB ? xs1 : xs0) + wave * kSlotX + xunit;
        uint32_t qlo = 0, qhi = 0, split = 8;
        float dsc0 = 0.0f, dsc1 = 0.0f;
        if constexpr (kNested) {
            if constexpr (kAligned) {
                if constexpr (QS == 2) {
                    qlo = jr.q.x >> (8u * jr.qinfo);     // the job's 2 bytes start at byte qf & 3
                } else {
                    qlo = jr.q.x;
                    qhi = jr.q.y;
                }
                const uint32_t d0 = jr.d[0];
                dsc0 = dsc1 = __builtin_bit_cast(float, d0);
            } else {
                const uint32_t sh = jr.qinfo & 3u;
                qlo = __builtin_amdgcn_alignbyte(jr.q[1], jr.q[0], sh);
                qhi = __builtin_amdgcn_alignbyte(jr.q[2], jr.q[1], sh);
                split = jr.qinfo >> 2;
                // (the elements go through plain locals: a bit cast of a vector element
                // lvalue reads the vector's first element)
                const uint32_t d0 = jr.d[0], d1 = jr.d[1];
                dsc0 = __builtin_bit_cast(float, d0);
                dsc1 = __builtin_bit_cast(float, d1);
            }
        }
        uint32_t fsel[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if constexpr (!kNested) {
            const u32x4_t f0 = jr.f0, f1 = jr.f1;
            fsel[0] = f0[0]; fsel[1] = f0[1]; fsel[2] = f0[2]; fsel[3] = f0[3];
            fsel[4] = f1[0]; fsel[5] = f1[1]; fsel[6] = f1[2]; fsel[7] = f1[3];
        }
        // the job's code words: row n, 16-weight group h of each of the 8 blocks (a plain
        // vector load: a copy of a HIP vector struct becomes a memcpy that loses the LDS
        // object's identity, and then every copy in flight is waited for)
        u32x2_t cwv[kChunkBlocks];
#pragma unroll
        for (int bb = 0; bb < kChunkBlocks; ++bb) {
            const int piece = 2 * bb + (h >> 1);
            cwv[bb] = *reinterpret_cast<const u32x2_t*>(mb + (16 * n + (piece ^ n)) * 16 + 8 * (h & 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the code reads have returned
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        refill();
        __builtin_amdgcn_sched_barrier(0);
        // block bb's table reads and x reads are issued before block bb - 1's MFMAs (two
        // register sets, alternating), so a block's LDS round trip overlaps the previous
        // block's work instead of stalling the wave once per block
        uint32_t wv[2][8];
        u32x4_t xv[2][2];
        auto fetch = [&](int bb) {
            const u32x2_t cw = cwv[bb];
            const uint32_t cws[2] = {cw[0], cw[1]};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    uint32_t addr = __builtin_amdgcn_perm(cws[t], lane_sel, 0x0C0C0400u | ((uint32_t)(4 + k4) << 8));
                    if constexpr (C == 32) addr >>= 1;
                    wv[bb & 1][4 * t + k4] = *reinterpret_cast<const uint32_t*>(tabb + addr);
                }
                xv[bb & 1][t] = xf[8 * bb + t];
            }
        };
        fetch(0);
#pragma unroll
        for (int bb = 0; bb < kChunkBlocks; ++bb) {
            if (bb + 1 < kChunkBlocks) fetch(bb + 1);
            __builtin_amdgcn_sched_barrier(0);
            floatx4_t pp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t* w = &wv[bb & 1][4 * t];
                pp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[bb & 1][t]),
                                                             __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3])),
                                                             pp, 0, 0, 0);
            }
            // the block's scale: quantization block bb >> QS of the job
            const uint32_t qq = (uint32_t)bb >> QS;
            float a;
            if constexpr (kNested) {
                const uint32_t word = qq < 4 ? qlo : qhi;
                const int32_t q8 = __builtin_amdgcn_sbfe((int32_t)word, 8 * (qq & 3), 8);
                const float dsc = qq < split ? dsc0 : dsc1;
                a = __fadd_rn(__fmul_rn((float)q8, dsc), c.mu);
            } else {
                a = __builtin_bit_cast(float, fsel[qq]);
            }
#pragma unroll
            for (int r = 0; r < kR; ++r) acc[r] = __builtin_fmaf(pp[r], a, acc[r]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    int32_t done = 0;          // tiles finished by this workgroup
    // the end of a tile: the wave's partial sums of the outputs m < M (registers r < M of
    // lanes 0..15) go to LDS; the S waves' partials are added after the last job, so the
    // waves never wait for each other inside the loop
    auto tile_end = [&]() {
        if (lane < 16) {
#pragma unroll
            for (int r = 0; r < kR; ++r) part[done][wave][r][lane] = acc[r];
        }
        acc = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
        ++done;
    };
    auto end_job = [&]() {
        if (cc.item < g.nitems && cc.j == cc.jobs - 1) tile_end();
        advance_comp(cc);
    };

    // jobs of each wave: the workgroup's tiles of each slice times its jobs per tile
    int32_t njobs = 0;
    for (int32_t t = 0; t < g.ntasks; ++t) {
        const int32_t lo = g.t[t].item0, hi = t + 1 < g.ntasks ? g.t[t + 1].item0 : g.nitems;
        const int32_t k0 = lo <= wg ? 0 : (lo - wg + G - 1) / G;   // first k with wg + k G >= lo
        const int32_t k1 = hi <= wg ? 0 : (hi - wg + G - 1) / G;   // first k with wg + k G >= hi
        njobs += (k1 - k0) * g.t[t].jobs;
    }

    using SlotA = std::integral_constant<bool, false>;
    using SlotB = std::integral_constant<bool, true>;
    using LoadAll = std::integral_constant<int, kLoadCodes | kLoadX>;
    using LoadCodes = std::integral_constant<int, kLoadCodes>;
    using LoadX = std::integral_constant<int, kLoadX>;
    JobRegs ra, rb;
    load(lc, ra, SlotA{}, LoadAll{});
    advance_load(lc);
    load(lc, rb, SlotB{}, LoadAll{});
    advance_load(lc);
    {
        // pair table: entry C b + copy for byte b.  Wave w writes the bytes b = w + S j,
        // whose nibbles are (j / (16 / S), w + S (j % (16 / S))); the level reads are
        // uniform (scalar loads), so they do not wait for the copies in flight
        constexpr int kLo = 16 / S;
        float lo[kLo];
#pragma unroll
        for (int q = 0; q < kLo; ++q) lo[q] = g.levels[wave + S * q];
        if (lane < C) {
#pragma unroll
            for (int jj = 0; jj < 256 / S; ++jj) {
                const float hi_nib = g.levels[jj / kLo];
                tab[(wave + S * jj) * C + lane] = pack_bf16x2(hi_nib, lo[jj % kLo]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the table is written; vmcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Two slots of jobs in flight.  Job j's scales and codes are issued at the start of job
    // j - 2's compute (as soon as that job's code words are in registers) and its x at the
    // end of it (once that job's x reads have returned), so the loads of a job issue in
    // the order scales + codes, x, and between job j's x and its compute only job j + 1's
    // kLoads loads are issued.  The loop runs whole pairs of jobs with no condition around a
    // load (the last pair may end with a job past the end, whose sums are never stored), has
    // no barrier and writes no global memory.
    //
    // The waits are explicit: before a job is computed, at most kLoads loads may still be in
    // flight (so every copy of this job has landed), and before a slot is refilled every LDS
    // read of it has returned.  (The compiler's own tracking of copies into LDS is not
    // relied on: it can miss the copies issued before the loop.)
    auto wait_job = [] {
        __builtin_amdgcn_s_waitcnt((kLoads & 15) | ((kLoads >> 4) << 14) | (7 << 4) | (15 << 8));
        asm volatile("" ::: "memory");
    };
    auto wait_lds = [] {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt untouched
        asm volatile("" ::: "memory");
    };
    const int32_t npairs = (njobs + 1) / 2;
    int32_t it = 0;
    do {
        wait_job();
        compute(cc, ra, SlotA{}, [&] { load(lc, ra, SlotA{}, LoadCodes{}); });
        wait_lds();
        load(lc, ra, SlotA{}, LoadX{});
        advance_load(lc);
        end_job();
        wait_job();
        compute(cc, rb, SlotB{}, [&] { load(lc, rb, SlotB{}, LoadCodes{}); });
        wait_lds();
        load(lc, rb, SlotB{}, LoadX{});
        advance_load(lc);
        end_job();
    } while (++it < npairs);

    // the last pair may have loaded jobs past the end: their copies into LDS land before
    // the workgroup ends
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    // outputs of the workgroup's tiles: the S partials added in wave order, to y
    int32_t t = 0;
    const int32_t per_pass = (S * 64) / (M * 16);   // tiles summed per pass of the workgroup
    for (int32_t k0 = 0; k0 < done; k0 += per_pass) {
        const int32_t k = k0 + (int32_t)threadIdx.x / (M * 16);
        const int e = (int)threadIdx.x % (M * 16);
        if ((int32_t)threadIdx.x < per_pass * M * 16 && k < done) {
            const int32_t item = wg + k * G;
            t = task_from(item, t);
            const GemvTask& T = g.t[t];
            const int64_t n0 = (int64_t)(item - T.item0) * 16;
            const int m = e >> 4, nn = e & 15;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < S; ++w) v += part[k][w][m][nn];
            if (n0 + nn < T.N) T.y[(int64_t)m * T.ystride + n0 + nn] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
        }
    }
}

// Swizzle of staged x row m in the row-split kernel.  A fragment read takes unit 8 b + 2 h
// + t of row min(n, M - 1) in lane (n, h); a 16-byte unit covers 4 of the 64 banks, so a
// row's units fall in 16 bank groups.  With up to 8 staged rows, bit 0 of m stays and
// bits 1 and 2 move to bits 2 and 3, so xswz(m) is in {0, 1, 4, 5, 8, 9, 12, 13}: the two
// h of a half wave (2 h in {0, 2} or {4, 6}) then reach 16 distinct groups, and the
// counters show no bank conflict at M = 4 and 8, where the plain m swizzle (which pairs
// row m of h with row m ^ 2 of h + 1) measured 0.7 conflict cycles per LDS instruction.
// With 16 staged rows the plain m swizzle measured no conflict and is kept.
template <int MX>
__device__ __forceinline__ int xswz(int m) {
    if constexpr (MX > 8) return m & 15;
    else return (m & 1) | ((m & 2) << 1) | ((m & 4) << 1);
}

// Row-split kernel for M >= 2 rows of x: each wave owns whole 16-row tiles and walks the
// row from k = 0 to K in 512-k jobs; the S waves of a workgroup own S consecutive tiles of
// one slice (a "group", one workgroup each, launched longest rows first so the hardware
// dispatcher balances them) and take the same job at the same time, so the x chunk of a
// job (M rows x 1 KB) is copied to LDS once per workgroup and shared.  Each wave's sums
// cover its whole rows, so the outputs go straight from registers to y.
//
// The codes and scales of a job are loaded two jobs ahead into the wave's own LDS slot
// and registers (as in the K-split kernel); the x chunk one job ahead into the shared
// slot, after the barrier that ends every wave's use of that slot.  x row m sits in its
// slot with its 16-byte units XOR-swizzled (unit u at u ^ xswz(m), the swizzle applied to
// the global offsets of the copy); see xswz for the bank groups of the fragment reads.
//
// kPair: the S waves own S / 2 tiles, two waves a tile, which take its even and its odd
// jobs; a step of the loop then covers two jobs (1024 k), whose x chunks the x slot holds
// side by side (row-chunk 2 m + c = chunk c of row m), and the two waves' sums are added
// through LDS at the end.  A workgroup then owns 64 rows, not 128: where one weight's rows
// are much longer than the others' (the down projection of a layer), the hardware
// dispatcher can balance the smaller workgroups over the CUs more evenly.
template <int S, int MX, bool kNested, int QS, bool kAligned, bool kPair>
__global__ __launch_bounds__(S * 64, 1) void gemv_rows_kernel(GemvGroup g) {
    constexpr int C = kTabCopies;
    constexpr int kJobQ = kChunkBlocks >> QS;
    constexpr int kLc = (kNested || QS == 0 ? 2 : 1) + 4;   // a job's scale loads and code copies
    constexpr int kTiles = kPair ? S / 2 : S;                 // tiles of a workgroup
    constexpr int kXC = kPair ? 2 * MX : MX;                  // row-chunks (1 KB each) of an x slot in use
    constexpr int kXL = (kXC + S - 1) / S;                    // row-chunks a wave copies per step
    constexpr int kXR = kXL * S;                              // row-chunks of an x slot (those >= kXC are never read)
    __shared__ __attribute__((aligned(4096))) uint32_t tab[256 * C];
    __shared__ __attribute__((aligned(1024))) uint4 cb0[S * 256];
    __shared__ __attribute__((aligned(1024))) uint4 cb1[S * 256];
    __shared__ __attribute__((aligned(1024))) uint4 xs0[kXR * 64];
    __shared__ __attribute__((aligned(1024))) uint4 xs1[kXR * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int h = lane >> 4;
    const int M = g.M;

    // this workgroup's group: slice t, tiles S (item - item0) + w
    const int32_t item = (int32_t)blockIdx.x;
    int32_t t = 0;
    while (t + 1 < g.ntasks && item >= g.t[t + 1].item0) ++t;
    const GemvTask& T = g.t[t];
    const int32_t N = (int32_t)T.N;
    const int32_t K = T.K;
    const int32_t nchunk = T.nchunk;
    const uint32_t row_bytes = (uint32_t)(K / 2);
    const int tw = kPair ? (wave & (kTiles - 1)) : wave;      // this wave's tile in the workgroup
    const int hf = kPair ? wave / kTiles : 0;                 // kPair: the wave takes jobs 2 i + hf
    const int32_t n0 = ((item - T.item0) * kTiles + tw) * 16;   // may be past N: rows clamped, never stored
    const float mu = kNested ? *(const __attribute__((address_space(4))) float*)(uintptr_t)T.dq_mean : 0.0f;
    const __amdgpu_buffer_rsrc_t cr = buf_rsrc(T.codes, T.code_bytes);
    const __amdgpu_buffer_rsrc_t xr = buf_rsrc(T.x, M * K * 2);
    const __amdgpu_buffer_rsrc_t sr = buf_rsrc(T.sc, T.sc_bytes);
    const __amdgpu_buffer_rsrc_t dr = buf_rsrc(T.dq_scale, T.dq_bytes);
    uint32_t crow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int32_t gr = n0 + r < N ? n0 + r : N - 1;
        crow[i] = (uint32_t)gr * row_bytes + 16u * (uint32_t)((lane & 15) ^ r);
    }
    const int32_t rowc = n0 + n < N ? n0 + n : N - 1;
    const uint32_t qrow = (uint32_t)T.qbase + (uint32_t)rowc * (uint32_t)(K >> (QS + 6));

    // codes and scales of job j (chunk clamped to the last: a job past the end reloads
    // valid memory and is never computed)
    auto load_codes = [&](int32_t j, JobRegs& jr, auto slot) {
        constexpr bool kB = decltype(slot)::value;
        const int32_t chc = j < nchunk ? j : nchunk - 1;
        const uint32_t qf = qrow + (uint32_t)(chc * kJobQ);
        if constexpr (kNested) {
            if constexpr (kAligned) {
                if constexpr (QS == 0)
                    jr.q.xy = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(sr, qrow, (uint32_t)(chc * kJobQ), 0));
                else
                    jr.q.x = __builtin_amdgcn_raw_buffer_load_b32(sr, qf & ~3u, 0, 0);
                if constexpr (QS == 2) jr.qinfo = qf & 3u;
                jr.d.x = __builtin_amdgcn_raw_buffer_load_b32(dr, (qf / QK_DQ_BLOCK) * 4u, 0, 0);
            } else {
                jr.q = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(sr, qf & ~3u, 0, 0));
                jr.d = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(dr, (qf / QK_DQ_BLOCK) * 4u, 0, 0));
                jr.qinfo = (qf & 3u) | ((QK_DQ_BLOCK - qf % QK_DQ_BLOCK) << 2);
            }
        } else {
            jr.f0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, qf * 4u, 0, 0));
            if constexpr (QS == 0)
                jr.f1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, qf * 4u + 16u, 0, 0));
        }
        __attribute__((address_space(3))) char* cdst =
            (__attribute__((address_space(3))) char*)reinterpret_cast<char*>(kB ? cb1 : cb0) + wave * 4096;
        const uint32_t cofs = (uint32_t)chc * (kChunkK / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t off = crow[i] + cofs;
            if constexpr (!kAligned) {
                // pieces past the end of a row (partial chunk) are clamped to its last 16 bytes
                const int r = 4 * i + (lane >> 4);
                const uint32_t piece = 16u * (uint32_t)((lane & 15) ^ r);
                off = cofs + piece + 16u <= row_bytes ? off : crow[i] + row_bytes - 16u - piece;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_ptr_t)(cdst + i * 1024), 16, off, 0, 0, kStream);
        }
    };
    // x row-chunks rc = wave + S i of step j (row m = rc, chunk j; kPair: row m = rc / 2,
    // chunk 2 j + rc % 2), unit L of the row from global unit L ^ m (k past the row in a
    // partial chunk, or a chunk past the row, reads zero).  Rows m >= M copy row M - 1 (they
    // feed only outputs that are never stored): every wave issues the same copies, with no
    // branch.
    uint32_t xo_live[kXL];
    auto load_x = [&](int32_t j, auto slot) {
        constexpr bool kB = decltype(slot)::value;
        __attribute__((address_space(3))) char* xdst =
            (__attribute__((address_space(3))) char*)reinterpret_cast<char*>(kB ? xs1 : xs0);
#pragma unroll
        for (int i = 0; i < kXL; ++i) {
            const int rc = wave + S * i;
            const int m = kPair ? rc >> 1 : rc;
            const int32_t ch = kPair ? 2 * j + (rc & 1) : j;
            const int ms = m < M ? m : M - 1;
            const int u = lane ^ xswz<MX>(m);
            const uint32_t xo = ch * kChunkK + 8 * u < K ? (uint32_t)(ch * (kChunkK * 2) + 16 * u + ms * K * 2) : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xdst + rc * 1024), 16, xo, 0, 0, 0);
            xo_live[i] = xo;
        }
    };
    // the offset registers of the x copies stay allocated until the job's reads are issued
    // (the compiler otherwise reuses one for an LDS read's result and waits for the copy)
    auto keep_x = [&] {
#pragma unroll
        for (int i = 0; i < kXL; ++i) asm volatile("" ::"v"(xo_live[i]));
    };

    floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t lane_sel = (uint32_t)lane * 4u;
    const char* tabb = reinterpret_cast<const char*>(tab);
    const int xrow = n < M ? n : M - 1;        // A operand rows m >= M: another row's data, never stored
    auto compute = [&](const JobRegs& jr, auto slot) {
        constexpr bool kB = decltype(slot)::value;
        const char* mb = reinterpret_cast<const char*>(kB ? cb1 : cb0) + wave * 4096;
        const u32x4_t* xf = reinterpret_cast<const u32x4_t*>(kB ? xs1 : xs0) + (kPair ? 2 * xrow + hf : xrow) * 64;
        uint32_t qlo = 0, qhi = 0, split = 8;
        float dsc0 = 0.0f, dsc1 = 0.0f;
        if constexpr (kNested) {
            if constexpr (kAligned) {
                if constexpr (QS == 2) {
                    qlo = jr.q.x >> (8u * jr.qinfo);
                } else {
                    qlo = jr.q.x;
                    qhi = jr.q.y;
                }
                const uint32_t d0 = jr.d[0];
                dsc0 = dsc1 = __builtin_bit_cast(float, d0);
            } else {
                const uint32_t sh = jr.qinfo & 3u;
                qlo = __builtin_amdgcn_alignbyte(jr.q[1], jr.q[0], sh);
                qhi = __builtin_amdgcn_alignbyte(jr.q[2], jr.q[1], sh);
                split = jr.qinfo >> 2;
                const uint32_t d0 = jr.d[0], d1 = jr.d[1];
                dsc0 = __builtin_bit_cast(float, d0);
                dsc1 = __builtin_bit_cast(float, d1);
            }
        }
#pragma unroll
        for (int bb = 0; bb < kChunkBlocks; ++bb) {
            const int piece = 2 * bb + (h >> 1);
            const u32x2_t cw = *reinterpret_cast<const u32x2_t*>(mb + (16 * n + (piece ^ n)) * 16 + 8 * (h & 1));
            const uint32_t cws[2] = {cw[0], cw[1]};
            floatx4_t pp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                uint32_t wv[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const uint32_t addr = __builtin_amdgcn_perm(cws[tt], lane_sel, 0x0C0C0400u | ((uint32_t)(4 + k4) << 8));
                    wv[k4] = *reinterpret_cast<const uint32_t*>(tabb + addr);
                }
                const u32x4_t xv = xf[(8 * bb + 2 * h + tt) ^ xswz<MX>(xrow)];
                pp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv),
                                                             __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3])),
                                                             pp, 0, 0, 0);
            }
            const uint32_t qq = (uint32_t)bb >> QS;
            float a;
            if constexpr (kNested) {
                const uint32_t word = qq < 4 ? qlo : qhi;
                const int32_t q8 = __builtin_amdgcn_sbfe((int32_t)word, 8 * (qq & 3), 8);
                const float dsc = qq < split ? dsc0 : dsc1;
                a = __fadd_rn(__fmul_rn((float)q8, dsc), mu);
            } else {
                const uint32_t fsel[8] = {jr.f0[0], jr.f0[1], jr.f0[2], jr.f0[3], jr.f1[0], jr.f1[1], jr.f1[2], jr.f1[3]};
                a = __builtin_bit_cast(float, fsel[qq]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(pp[r], a, acc[r]);
        }
    };

    using SlotA = std::integral_constant<bool, false>;
    using SlotB = std::integral_constant<bool, true>;
    JobRegs ra, rb;
    // the job of this wave in step j, and the steps
    auto cj = [&](int32_t j) { return kPair ? 2 * j + hf : j; };
    const int32_t nsteps = kPair ? (nchunk + 1) / 2 : nchunk;
    // issue order codes(0), x(0), codes(1): the wait before step j allows only the codes of
    // step j + 1 in flight
    load_codes(cj(0), ra, SlotA{});
    load_x(0, SlotA{});
    load_codes(cj(1), rb, SlotB{});
    {
        constexpr int kLo = 16 / S;
        float lo[kLo];
#pragma unroll
        for (int q = 0; q < kLo; ++q) lo[q] = g.levels[wave + S * q];
        if (lane < C) {
#pragma unroll
            for (int jj = 0; jj < 256 / S; ++jj) {
                const float hi_nib = g.levels[jj / kLo];
                tab[(wave + S * jj) * C + lane] = pack_bf16x2(hi_nib, lo[jj % kLo]);
            }
        }
    }
    // (each wait is also a scheduling barrier: the compiler would otherwise hoist the next
    // job's scale arithmetic above it and wait for that job's loads)
    auto wait_job = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((kLc & 15) | ((kLc >> 4) << 14) | (7 << 4) | (15 << 8));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto wait_lds = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt untouched
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // Job j: wait until this wave's codes and x part of job j have landed (only the codes of
    // job j + 1 may be in flight), and the table is written; the barrier then makes every
    // wave's x part visible and ends every wave's reads of the other x slot, which takes
    // job j + 1's x; after the job, its code slot takes job j + 2.  The loop runs whole pairs
    // of jobs with no condition around a load or a read (a condition makes the compiler
    // wait for every copy in flight): a job past the end reads x as zero and adds nothing.
    for (int32_t j = 0; j < nsteps; j += 2) {
        wait_job();
        wait_lds();
        barrier();
        load_x(j + 1, SlotB{});
        compute(ra, SlotA{});
        keep_x();
        wait_lds();
        load_codes(cj(j + 2), ra, SlotA{});
        wait_job();
        barrier();
        load_x(j + 2, SlotA{});
        compute(rb, SlotB{});
        keep_x();
        wait_lds();
        load_codes(cj(j + 3), rb, SlotB{});
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no copy into LDS outlives the workgroup
    if constexpr (kPair) {
        // the odd jobs' sums go through the wave's own code slot to the wave of the even
        // jobs, which adds them to its own (in that order) and stores the tile
        floatx4_t* mine = reinterpret_cast<floatx4_t*>(reinterpret_cast<char*>(cb0) + wave * 4096) + lane;
        if (hf == 1) *mine = acc;
        __syncthreads();
        if (hf == 1) return;
        const floatx4_t other = *reinterpret_cast<const floatx4_t*>(reinterpret_cast<const char*>(cb0) +
                                                                    (wave + kTiles) * 4096 + 16 * lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += other[r];
    }
    // outputs: register r of lane l is y[4 (l / 16) + r][n0 + l % 16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * h + r;
        if (m < M && n0 + n < N)
            T.y[(int64_t)m * T.ystride + n0 + n] = (uint16_t)(pack_bf16x2(acc[r], 0.0f) & 0xFFFFu);
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

hipError_t launch_gemv_group(const GemvItem* items, int32_t count, int32_t M, hipStream_t s,
                             const char** variant) {
    // M = 1: the K-split kernel (8 waves share each 16-row tile, persistent); M >= 2: the
    // row-split kernel (8 waves, one 16-row tile each, sharing the x chunk; one workgroup
    // per group of 8 tiles)
    const bool rows = M >= kRowsMinM;
    const int S = 8;
    const int MX = rows ? (M <= 4 ? 4 : M <= 8 ? 8 : 16) : 1;
    // row-split: two waves a tile (4 tiles a workgroup) at M <= 4, else one (8 tiles).  On
    // the 70B-shaped layer (M = 4) the pairs took 120 us against 124 (alternating runs on
    // one GPU); at M = 8, where a step copies 16 KB of x, they were no faster.
    const bool pair = rows && MX == 4;
    const int tiles_per_wg = pair ? S / 2 : S;
    const int64_t cus = device_cu_count();
    // tiles per launch: the K-split kernel's LDS holds each workgroup's partials; the
    // row-split kernel's groups are only bounded by the grid
    const int64_t max_tiles = rows ? ((int64_t)1 << 30) : (int64_t)out_slots(S, MX) * cus;
    // weights the fast kernel cannot take go one by one through the generic kernel; the
    // others are cut into slices of rows whose codes fit a 31-bit buffer offset and whose
    // tiles fit one launch
    std::vector<GemvTask> slices;
    std::vector<const DeqArgs*> slice_w;
    for (int32_t i = 0; i < count; ++i) {
        const MatArgs& w = items[i].w;
        const int64_t nb = (w.N * w.K) >> w.w.blocksize_log2;
        const bool ok = (w.K % kStep) == 0 && (w.K % w.w.blocksize) == 0 &&
                        (reinterpret_cast<uintptr_t>(items[i].x) % 16) == 0 &&
                        (reinterpret_cast<uintptr_t>(w.w.codes) % 16) == 0 && (int64_t)M * w.K * 2 < ((int64_t)1 << 31) &&
                        w.K / 2 * 16 < ((int64_t)1 << 31) && (w.w.nested ? nb : 4 * nb) < ((int64_t)1 << 31);
        if (!ok) {
            GemvArgs a;
            a.x = reinterpret_cast<const uint16_t*>(items[i].x);
            a.y = reinterpret_cast<uint16_t*>(items[i].y);
            a.w = w.w;
            a.N = w.N;
            a.K = w.K;
            a.M = M;
            *variant = "generic (per-element dequantization, one wave per row)";
            hipLaunchKernelGGL(gemv_generic_kernel, dim3((unsigned)((w.N + 3) / 4)), dim3(256), 0, s, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }
        int64_t rows = (((int64_t)1 << 31) - 1) / (w.K / 2);
        rows = rows < max_tiles * 16 ? rows : max_tiles * 16;
        rows -= rows % 16;
        for (int64_t r0 = 0; r0 < w.N; r0 += rows) {
            GemvTask t{};
            const int64_t nr = w.N - r0 < rows ? w.N - r0 : rows;
            t.x = reinterpret_cast<const uint16_t*>(items[i].x);
            t.y = reinterpret_cast<uint16_t*>(items[i].y) + r0;
            t.codes = w.w.codes + r0 * (w.K / 2);
            t.sc = w.w.nested ? static_cast<const void*>(w.w.q8) : static_cast<const void*>(w.w.absmax);
            t.dq_scale = w.w.dq_scale;
            t.dq_mean = w.w.dq_mean;
            t.N = nr;
            t.ystride = w.N;
            t.qbase = (r0 * w.K) >> w.w.blocksize_log2;
            t.K = (int32_t)w.K;
            t.nchunk = (int32_t)((w.K + kChunkK - 1) / kChunkK);
            t.jobs = (t.nchunk + S - 1) / S;
            t.code_bytes = (int32_t)(nr * (w.K / 2));
            // buffer loads check their range per dword and return zero for a dword that ends
            // past it: the q8 range is rounded up to whole dwords so the last q8 bytes read
            // back (the up to 3 bytes after the array share its last dword, and so its page;
            // they are never used)
            t.sc_bytes = (int32_t)(w.w.nested ? (nb + 3) / 4 * 4 : 4 * nb);
            t.dq_bytes = (int32_t)(w.w.nested ? 4 * ((nb + QK_DQ_BLOCK - 1) / QK_DQ_BLOCK) : 0);
            slices.push_back(t);
            slice_w.push_back(&w.w);
        }
    }
    // launches of slices that share the code table, block size and nesting, longest rows
    // first (a workgroup takes tiles blockIdx.x, + grid, ...: the long tiles are spread
    // over the workgroups before the short ones)
    std::vector<size_t> order(slices.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return slices[a].K > slices[b].K; });
    std::vector<bool> used(slices.size(), false);
    for (size_t f = 0; f < order.size(); ++f) {
        if (used[order[f]]) continue;
        const DeqArgs& w0 = *slice_w[order[f]];
        // rows that are whole jobs take the kernel whose scales are one aligned run per job;
        // a weight whose rows are not puts the whole group on the general variant rather
        // than costing a launch of its own
        bool aligned = true;
        for (size_t f2 = f; f2 < order.size(); ++f2) {
            const size_t k = order[f2];
            const DeqArgs& w = *slice_w[k];
            if (!used[k] && w.nested == w0.nested && w.blocksize == w0.blocksize &&
                std::memcmp(w.levels, w0.levels, sizeof(w.levels)) == 0 && slices[k].K % kChunkK != 0)
                aligned = false;
        }
        GemvGroup gg;
        std::memset(&gg, 0, sizeof(gg));
        std::memcpy(gg.levels, w0.levels, sizeof(gg.levels));
        gg.M = M;
        int64_t nitems = 0;
        for (size_t f2 = f; f2 < order.size() && gg.ntasks < kMaxGemvTasks; ++f2) {
            const size_t k = order[f2];
            if (used[k]) continue;
            const DeqArgs& w = *slice_w[k];
            if (w.nested != w0.nested || w.blocksize != w0.blocksize ||
                std::memcmp(w.levels, w0.levels, sizeof(w.levels)) != 0)
                continue;
            // an aligned launch takes only weights whose rows are whole jobs
            if (aligned && slices[k].K % kChunkK != 0) continue;
            const int64_t tiles = (slices[k].N + 15) / 16;
            const int64_t units = rows ? (tiles + tiles_per_wg - 1) / tiles_per_wg : tiles;   // row-split: groups of tiles
            if (nitems + units > max_tiles) continue;
            GemvTask& t = gg.t[gg.ntasks++];
            t = slices[k];
            t.item0 = (int32_t)nitems;
            nitems += units;
            used[k] = true;
        }
        gg.nitems = (int32_t)nitems;
        gg.qs = w0.blocksize_log2 - 6;
        const unsigned grid = rows ? (unsigned)nitems : (unsigned)(nitems < cus ? nitems : cus);
        *variant = pair ? "mfma 16x16x32 bf16, row-split grouped launch: one workgroup per 4 tiles of 16 rows, two waves "
                          "a tile (even and odd 512-k jobs), the x chunks shared through LDS, codes and scales two steps ahead"
                 : rows ? "mfma 16x16x32 bf16, row-split grouped launch: one workgroup per 8 tiles of 16 rows, each wave "
                          "a whole tile, the x chunk shared through LDS, codes and scales two 512-k jobs ahead"
                        : "mfma 16x16x32 bf16, persistent grouped launch: 16-row tiles split over 8 waves in 512-k jobs, "
                          "two jobs in flight per wave, codes and x copied to LDS";
        if (rows) {
#define QK_GEMV_ROWS_A(MXX, NN, QQ)                                                                                    \
    do {                                                                                                               \
        if (aligned) hipLaunchKernelGGL((gemv_rows_kernel<8, MXX, NN, QQ, true, (MXX == 4)>), dim3(grid), dim3(8 * 64), 0, s, gg); \
        else hipLaunchKernelGGL((gemv_rows_kernel<8, MXX, NN, QQ, false, (MXX == 4)>), dim3(grid), dim3(8 * 64), 0, s, gg);        \
    } while (0)
#define QK_GEMV_ROWS_Q(MXX, QQ)                                  \
    do {                                                         \
        if (w0.nested) QK_GEMV_ROWS_A(MXX, true, QQ);            \
        else QK_GEMV_ROWS_A(MXX, false, QQ);                     \
    } while (0)
#define QK_GEMV_ROWS(MXX)                                        \
    do {                                                         \
        if (gg.qs == 0) QK_GEMV_ROWS_Q(MXX, 0);                  \
        else if (gg.qs == 1) QK_GEMV_ROWS_Q(MXX, 1);             \
        else QK_GEMV_ROWS_Q(MXX, 2);                             \
    } while (0)
            if (MX == 4) QK_GEMV_ROWS(4);
            else if (MX == 8) QK_GEMV_ROWS(8);
            else QK_GEMV_ROWS(16);
#undef QK_GEMV_ROWS
#undef QK_GEMV_ROWS_Q
#undef QK_GEMV_ROWS_A
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }
#define QK_GEMV_LAUNCH_A(SS, MXX, CC, NN, QQ)                                                                      \
    do {                                                                                                           \
        if (aligned) hipLaunchKernelGGL((gemv_group_kernel<SS, MXX, CC, NN, QQ, true>), dim3(grid), dim3(SS * 64), 0, s, gg); \
        else hipLaunchKernelGGL((gemv_group_kernel<SS, MXX, CC, NN, QQ, false>), dim3(grid), dim3(SS * 64), 0, s, gg); \
    } while (0)
#define QK_GEMV_LAUNCH_Q(SS, MXX, CC, QQ)                                \
    do {                                                                 \
        if (w0.nested) QK_GEMV_LAUNCH_A(SS, MXX, CC, true, QQ);          \
        else QK_GEMV_LAUNCH_A(SS, MXX, CC, false, QQ);                   \
    } while (0)
#define QK_GEMV_LAUNCH(SS, MXX, CC)                       \
    do {                                                  \
        if (gg.qs == 0) QK_GEMV_LAUNCH_Q(SS, MXX, CC, 0); \
        else if (gg.qs == 1) QK_GEMV_LAUNCH_Q(SS, MXX, CC, 1); \
        else QK_GEMV_LAUNCH_Q(SS, MXX, CC, 2);            \
    } while (0)
        QK_GEMV_LAUNCH(8, 1, 64);
#undef QK_GEMV_LAUNCH
#undef QK_GEMV_LAUNCH_Q
#undef QK_GEMV_LAUNCH_A
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv(const void* x, int32_t M, const MatArgs& w, void* y, hipStream_t s, const char** variant) {
    const GemvItem it{x, y, w};
    return launch_gemv_group(&it, 1, M, s, variant);
}

}  // namespace qk
