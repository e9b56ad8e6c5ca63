// HBM ceilings for the measurement script (not part of the qk C ABI): a grid of
// 256-thread workgroups streams a buffer with 16-byte loads, 16 per lane in flight,
// plain or with the nontemporal hint, and folds the words into one value per thread so
// that no load is dropped; two mixed streams read and write in the proportions of the
// quantization and of the dequantization.  bench.py times them with HIP events next to
// a device copy.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 16;

template <bool kNontemporal>
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4_t* __restrict__ p, size_t n16,
                                                               uint32_t* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride * kUnroll) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t k = i + (size_t)j * stride;
            if (k < n16) v[j] = kNontemporal ? __builtin_nontemporal_load(p + k) : p[k];
            else v[j] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

// Reads nbytes (a multiple of 16, 16-byte aligned) at src; out holds grid * 256 words.
// Returns 0, or a nonzero code for bad arguments or a failed launch.
extern "C" int qk_probe_read_stream(const void* src, size_t nbytes, uint32_t* out, int grid, int nontemporal,
                                    void* stream) {
    if (src == nullptr || out == nullptr || nbytes == 0 || nbytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(src) % 16 != 0 || grid <= 0)
        return 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4_t* p = static_cast<const u32x4_t*>(src);
    if (nontemporal)
        hipLaunchKernelGGL(read_stream_kernel<true>, dim3(grid), dim3(kThreads), 0, s, p, nbytes / 16, out);
    else
        hipLaunchKernelGGL(read_stream_kernel<false>, dim3(grid), dim3(kThreads), 0, s, p, nbytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Mixed streams: kReadHeavy reads 16 bytes (nontemporal) and writes 4 per lane and
// step (the traffic of a 4-bit quantization of 16-bit input: 2 bytes in, about half a
// byte out); otherwise it reads 4 bytes and writes 16 (a dequantization to 16 bits).
namespace {

constexpr int kMixUnroll = 8;

// kMode 0: read-heavy, 4-byte stores; 1: write-heavy; 2: read-heavy, the words of 4
// neighbouring lanes gathered by DPP into one 16-byte store (n16 a multiple of 4)
template <int kMode>
__global__ __launch_bounds__(kThreads) void mix_stream_kernel(const void* __restrict__ src, void* __restrict__ dst,
                                                              size_t n16) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride * kMixUnroll) {
        if constexpr (kMode != 1) {
            u32x4_t v[kMixUnroll];
#pragma unroll
            for (int j = 0; j < kMixUnroll; ++j) {
                const size_t k = i + (size_t)j * stride;
                v[j] = k < n16 ? __builtin_nontemporal_load(static_cast<const u32x4_t*>(src) + k) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < kMixUnroll; ++j) {
                const size_t k = i + (size_t)j * stride;
                const uint32_t w = v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
                if constexpr (kMode == 0) {
                    if (k < n16) static_cast<uint32_t*>(dst)[k] = w;
                } else {
                    // k and the grid's lane count are multiples of 4 at lanes 4 q, so the
                    // quad's 4 steps are k .. k + 3, all in range or all out
                    const uint32_t w1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x39, 0xF, 0xF, false);   // lane + 1
                    const uint32_t w2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x4E, 0xF, 0xF, false);   // lane + 2
                    const uint32_t w3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x93, 0xF, 0xF, false);   // lane + 3
                    if ((threadIdx.x & 3) == 0 && k < n16) static_cast<u32x4_t*>(dst)[k / 4] = u32x4_t{w, w1, w2, w3};
                }
            }
        } else {
            uint32_t w[kMixUnroll];
#pragma unroll
            for (int j = 0; j < kMixUnroll; ++j) {
                const size_t k = i + (size_t)j * stride;
                w[j] = k < n16 ? static_cast<const uint32_t*>(src)[k] : 0u;
            }
#pragma unroll
            for (int j = 0; j < kMixUnroll; ++j) {
                const size_t k = i + (size_t)j * stride;
                if (k < n16) static_cast<u32x4_t*>(dst)[k] = u32x4_t{w[j], w[j] ^ 1u, w[j] ^ 2u, w[j] ^ 3u};
            }
        }
    }
}

}  // namespace

// n16 steps of 16 bytes: read_heavy != 0 reads 16 n16 bytes at src and writes 4 n16 at
// dst (read_heavy = 2: by 16-byte stores, n16 a multiple of 4); otherwise reads 4 n16
// and writes 16 n16.  Both buffers 16-byte aligned.  Returns 0,
// or a nonzero code for bad arguments or a failed launch.
extern "C" int qk_probe_mix_stream(const void* src, void* dst, size_t n16, int grid, int read_heavy, void* stream) {
    if (src == nullptr || dst == nullptr || n16 == 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0 || grid <= 0)
        return 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (read_heavy == 2 && n16 % 4 != 0) return 1;
    if (read_heavy == 2)
        hipLaunchKernelGGL(mix_stream_kernel<2>, dim3(grid), dim3(kThreads), 0, s, src, dst, n16);
    else if (read_heavy)
        hipLaunchKernelGGL(mix_stream_kernel<0>, dim3(grid), dim3(kThreads), 0, s, src, dst, n16);
    else
        hipLaunchKernelGGL(mix_stream_kernel<1>, dim3(grid), dim3(kThreads), 0, s, src, dst, n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Row-block streams of a row-major [M, K] bf16 matrix, the access pattern of a pass
// that takes 16 rows per wave, 4 waves per workgroup and K in nsplit splits, one
// 64-element step at a time, 4 steps in flight per lane.  kFullLines 0: lane
// (row l % 16, quarter l / 16) loads 16 bytes at 16 q and 64 + 16 q of its row (each
// load instruction takes half of 16 lines); 1: a load instruction takes 8 whole 128-byte
// lines (lane l: row 8 i + l / 8, bytes 16 (l % 8)); 2: the same 8 whole lines with the
// lanes in the other order (lane l: row 8 i + l % 8, bytes 16 (l / 8)), so consecutive
// lanes read different rows.  Reads are folded into one word per thread.
namespace {

template <int kFullLines>
__global__ __launch_bounds__(256) void rowblock_stream_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                              int nsplit, uint32_t* __restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nrb = (M + 63) / 64;
    const int64_t rb = blockIdx.x % nrb, split = blockIdx.x / nrb;
    const int64_t nk = K / 64, s0 = nk * split / nsplit, s1 = nk * (split + 1) / nsplit;
    int64_t r0, r1, c0, c1;
    if constexpr (kFullLines == 1) {
        r0 = rb * 64 + 16 * wave + lane / 8;
        r1 = r0 + 8;
        c0 = c1 = 8 * (lane % 8);
    } else if constexpr (kFullLines == 2) {
        r0 = rb * 64 + 16 * wave + lane % 8;
        r1 = r0 + 8;
        c0 = c1 = 8 * (lane / 8);
    } else {
        r0 = r1 = rb * 64 + 16 * wave + (lane & 15);
        c0 = 8 * (lane >> 4);
        c1 = c0 + 32;
    }
    r0 = r0 < M ? r0 : M - 1;
    r1 = r1 < M ? r1 : M - 1;
    uint32_t acc = 0;
    u32x4_t v[4][2];
    auto ld = [&](int64_t s, u32x4_t (&d)[2]) {
        const int64_t sc = s < s1 ? s : s1 - 1;
        d[0] = *reinterpret_cast<const u32x4_t*>(x + r0 * K + sc * 64 + c0);
        d[1] = *reinterpret_cast<const u32x4_t*>(x + r1 * K + sc * 64 + c1);
    };
    if (s0 < s1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ld(s0 + i, v[i]);
        for (int64_t s = s0; s < s1; s += 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc ^= v[i][0].x ^ v[i][0].y ^ v[i][0].z ^ v[i][0].w ^ v[i][1].x ^ v[i][1].y ^ v[i][1].z ^ v[i][1].w;
                __builtin_amdgcn_sched_barrier(0);
                ld(s + 4 + i, v[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    out[(int64_t)blockIdx.x * 256 + tid] = acc;
}

}  // namespace

// Streams x [M, K] bf16 (K a multiple of 64, x 16-byte aligned) in the row-block
// pattern above; out holds ceil(M / 64) * nsplit * 256 words.  Returns 0, or a nonzero
// code for bad arguments or a failed launch.
extern "C" int qk_probe_rowblock_stream(const void* x, int64_t M, int64_t K, int nsplit, int full_lines,
                                        uint32_t* out, void* stream) {
    if (x == nullptr || out == nullptr || M < 1 || K < 64 || K % 64 != 0 || nsplit < 1 || nsplit > K / 64 ||
        full_lines < 0 || full_lines > 2 ||
        reinterpret_cast<uintptr_t>(x) % 16 != 0)
        return 1;
    const dim3 grid((unsigned)(((M + 63) / 64) * nsplit));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* p = static_cast<const uint16_t*>(x);
    if (full_lines == 2)
        hipLaunchKernelGGL(rowblock_stream_kernel<2>, grid, dim3(256), 0, s, p, M, K, nsplit, out);
    else if (full_lines == 1)
        hipLaunchKernelGGL(rowblock_stream_kernel<1>, grid, dim3(256), 0, s, p, M, K, nsplit, out);
    else
        hipLaunchKernelGGL(rowblock_stream_kernel<0>, grid, dim3(256), 0, s, p, M, K, nsplit, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The range check of a raw buffer load that writes into LDS: one wave, 64 lanes,
// lane l loads 16 bytes at vector offset 16 l and the given scalar offset from a
// resource of num_records = 512 bytes at src (which must hold at least 512 +
// soffset bytes so that every address stays in the allocation); out[4 l .. 4 l + 4)
// receives what landed in LDS.  Lanes whose vector + scalar offset reach 512 read
// zero where the scalar offset takes part in the check.
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(64) void buffer_range_kernel(const uint32_t* src, uint32_t* out, uint32_t soffset) {
    __shared__ __attribute__((aligned(16))) uint32_t buf[256];
    const int lane = threadIdx.x;
    for (int i = 0; i < 4; ++i) buf[4 * lane + i] = 0xFFFFFFFFu;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(src), (short)0, 512, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)buf, 16, 16u * (uint32_t)lane, soffset, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    for (int i = 0; i < 4; ++i) out[4 * lane + i] = buf[4 * lane + i];
}

}  // namespace

extern "C" int qk_probe_buffer_range(const void* src, size_t src_bytes, uint32_t* out, uint32_t soffset,
                                     void* stream) {
    if (src == nullptr || out == nullptr || soffset % 16 != 0 || src_bytes < 512 + (size_t)soffset + 1024)
        return 1;
    hipLaunchKernelGGL(buffer_range_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(src), out, soffset);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
