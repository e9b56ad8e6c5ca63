// Internal declarations shared by the host API and the HIP kernels of libqk.
// Not installed; the public ABI is include/qk.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qk.h"

namespace qk {

// ---------------------------------------------------------------------------
// Exact nearest-level lookup used by the quantize kernel.
//
// The normalised value t lies in [-1, 1].  It is binned by
//     bin(t) = RN(t * S + S)   (an integer in [0, 2S], computed as the low 24
//                                bits of fmaf(t, S, S + 2^23))
// which is monotone in t.  The host evaluates the same fmaf, finds in which bin
// every decision threshold falls, and checks that no bin holds two.  Each bin
// then stores the code below its threshold, the code above it, and the
// threshold itself (a binary32 value T such that "t >= T" is exactly the
// nearest-level decision, tie rule included).  A bin without a threshold
// stores T = 2 (never reached).
// ---------------------------------------------------------------------------
constexpr int kLutMaxS = 64;
constexpr int kLutMaxBins = 2 * kLutMaxS + 1;

struct QuantLut {
    float S;                 // bins per unit of t
    float C;                 // S + 2^23
    int32_t nbins;           // 2S + 1
    int32_t sorted;          // 1: code order is value order (codes are c_lo + [t >= T])
    int32_t tiny_free;       // 1: no threshold in (-2^-60, 2^-60], so every |t| < 2^-60 gets one code
    float T[kLutMaxBins];    // threshold of each bin
    uint32_t c[kLutMaxBins]; // sorted: c_lo; otherwise c_lo | (c_hi << 16)
};

// Build the lookup for a level table (code order).  Returns QK_OK,
// QK_ERR_INVALID_ARG (non-finite or out of [-1, 1]) or QK_ERR_UNSUPPORTED (a
// midpoint that is not exact in binary64, or thresholds too close for S <= 64).
qk_status build_quant_lut(const float levels[16], QuantLut* lut, const char** why);

// ---------------------------------------------------------------------------
// 8-bit quantization (256 levels).  The same exact decision as above, but the
// per-bin table (up to 2049 bins) is too large for kernel arguments: the host
// passes the sorted thresholds and the code of each sorted value, validated to
// put at most one threshold in any bin of width 1/S, and each workgroup builds
// the bin table in LDS.  With S a power of two, bin(t) = round-half-even(t S + S),
// so the least t of bin b is (b - S - 1/2) / S when b is even and the next binary32
// value above it when b is odd.
// ---------------------------------------------------------------------------
constexpr int kLut8MaxS = 1024;
constexpr int kLut8MaxBins = 2 * kLut8MaxS + 1;

struct QuantLut8 {
    float S;                 // bins per unit of t (power of two)
    float C;                 // S + 2^23
    int32_t nbins;           // 2S + 1
    int32_t nthr;            // distinct level values - 1
    float T[255];            // increasing: t >= T[s] puts t above the s-th smallest value
    uint8_t code_of[256];    // smallest code carrying the s-th smallest value
};

qk_status build_quant_lut8(const float levels[256], QuantLut8* lut, const char** why);
// Dynamic 8-bit map: 256 equal-mass quantiles of N(0, 1) (signed) or of |N(0, 1)|
// (unsigned), divided by the largest.
qk_status make_dynamic_map(int32_t is_signed, float out[256]);

// Level tables.
qk_status make_nf4(float out[16]);
qk_status make_fp4(float out[16]);

// Standard normal quantile, Wichura's algorithm AS 241 (PPND16), fp64.
double normal_quantile(double p);

// Compute units of the current device (cached; 256 if the query fails).
int device_cu_count();

// ---------------------------------------------------------------------------
// Kernel launchers (return hipError_t of the launch).
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize,
                           const QuantLut& lut, uint8_t* codes, float* absmax, hipStream_t s);
// one array of a grouped quantization (same dtype, block size and level table for all)
struct QuantItem {
    const void* x;
    int64_t n;
    uint8_t* codes;
    float* absmax;
};
hipError_t launch_quantize_group(const QuantItem* items, int32_t count, int32_t x_dtype, int32_t blocksize,
                                 const QuantLut& lut, hipStream_t s);

hipError_t launch_quantize8(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize, const QuantLut8& lut,
                            uint8_t* codes, float* absmax, hipStream_t s);
hipError_t launch_dequantize8(const uint8_t* codes, const float* absmax, int64_t n, int32_t blocksize,
                              const float levels[256], void* out, int32_t out_dtype, hipStream_t s);

hipError_t launch_int8_rowquant(const void* x, int32_t dtype, int64_t rows, int64_t cols, const uint8_t* skip,
                                int8_t* q, float* absmax, hipStream_t s);
hipError_t launch_int8_outliers(const void* x, int32_t dtype, int64_t M, int64_t K, float threshold, float* colmax,
                                uint8_t* flags, int32_t* idx, int32_t* count, hipStream_t s);
hipError_t launch_int8_matmul(const int8_t* Xq, const float* SX, const int8_t* CB, const float* SCB, int64_t M,
                              int64_t N, int64_t K, const void* X, const int32_t* oidx, const int32_t* ocount, void* Y,
                              hipStream_t s);

size_t dq_workspace_bytes(int64_t nblocks);
hipError_t launch_double_quant(const float* absmax, int64_t nblocks, int8_t* q8, float* scale,
                               float* mean, void* workspace, hipStream_t s);
// one array of a grouped double quantization
struct DqItem {
    const float* absmax;
    int64_t nblocks;
    int8_t* q8;
    float* scale;
    float* mean;
};
// workspace: the items' dq_workspace_bytes() back to back, in item order
hipError_t launch_double_quant_group(const DqItem* items, int32_t count, void* workspace, hipStream_t s);

struct DeqArgs {
    const uint8_t* codes;
    const float* absmax;
    const int8_t* q8;
    const float* dq_scale;
    const float* dq_mean;
    int64_t n;
    int32_t blocksize;
    int32_t blocksize_log2;  // blocksize is a power of two: block of element e = e >> blocksize_log2
    int32_t nested;
    float levels[16];
};
hipError_t launch_dequantize(const DeqArgs& a, void* out, int32_t out_dtype, hipStream_t s);
// one array of a grouped dequantization
struct DeqItem {
    DeqArgs a;
    void* out;
};
hipError_t launch_dequantize_group(const DeqItem* items, int32_t count, int32_t out_dtype, hipStream_t s);

struct MatArgs {
    DeqArgs w;       // the weight [N, K]
    int64_t N;
    int64_t K;
};
hipError_t launch_gemv(const void* x, int32_t M, const MatArgs& w, void* y, hipStream_t s,
                       const char** variant);
// Several weights with their own x and y (the same M) in as few launches as their
// code tables, block sizes and nesting allow (at most kMaxGemvTasks weights each).
constexpr int kMaxGemvTasks = 16;
struct GemvItem {
    const void* x;
    void* y;
    MatArgs w;
};
hipError_t launch_gemv_group(const GemvItem* items, int32_t count, int32_t M, hipStream_t s,
                             const char** variant);
size_t gemm_workspace_bytes(int64_t M, int32_t r);
// The static device scratch of the no-allocation GEMM: its size, and its address
// on the current device (looked up with hipGetSymbolAddress on the first call per
// device, then cached).
size_t gemm_noalloc_scratch_bytes();
hipError_t gemm_noalloc_scratch(void** ptr);
// One GEMM of a grouped call.
struct GemmItem {
    const void* X;
    int64_t M;
    MatArgs w;
    const void* A;
    const void* B;
    int32_t r;
    float lora_scale;
    void* Y;
};
size_t gemm_group_workspace_bytes(const GemmItem* items, int32_t count);
hipError_t launch_gemm_group(const GemmItem* items, int32_t count, void* workspace, hipStream_t s,
                             const char** variant);
hipError_t launch_gemm(const void* X, int64_t M, const MatArgs& w, const void* A, const void* B,
                       int32_t r, float lora_scale, void* Y, void* workspace, hipStream_t s,
                       const char** variant);

// s * X * A in fp32 ([M, 16 * ceil(r / 16)], ranks >= r zero): K % 64 == 0, X 16-byte
// aligned; T_splits holds the per-K-split partials (gemm_workspace_bytes(M, r) bytes).
hipError_t launch_lora_xa_sum(const void* X, int64_t M, int64_t K, const void* A, int32_t r, float lora_scale,
                              float* T_splits, float* Ts, hipStream_t s);
size_t qlora_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r);
hipError_t launch_qlora_backward(const void* dY, int64_t M, const MatArgs& w, const void* X, const void* A,
                                 const void* B, int32_t r, float lora_scale, void* dX, float* dA, float* dB,
                                 void* workspace, hipStream_t s);
hipError_t launch_lora_merge(const MatArgs& w, const void* A, const void* B, int32_t r, float scale, void* out,
                             hipStream_t s);

}  // namespace qk
