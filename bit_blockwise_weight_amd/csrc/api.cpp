// C ABI of libqk: argument and descriptor validation, error reporting, kernel
// launch.  Every check runs on the host before anything is launched and no
// device pointer is dereferenced here; a rejected call launches nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qk_internal.h"

namespace {

thread_local std::string g_last_error;

qk_status ok() {
    g_last_error.clear();
    return QK_OK;
}

qk_status fail(qk_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_blocksize(int32_t b) { return b == 64 || b == 128 || b == 256; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The current device must be a gfx950 (checked once per device id).
qk_status ensure_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return fail(QK_ERR_NO_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    static int checked[64] = {0};   // 0 unknown, 1 ok, 2 wrong arch
    if (dev < 64 && checked[dev] == 1) return QK_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(QK_ERR_NO_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) checked[dev] = good ? 1 : 2;
    if (!good) return fail(QK_ERR_NO_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
    return QK_OK;
}

qk_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(QK_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

qk_status validate_state(const qk_quant_state* st) {
    if (!st) return fail(QK_ERR_INVALID_ARG, "quant state pointer is NULL");
    if (st->magic != QK_STATE_MAGIC)
        return fail(QK_ERR_BAD_STATE, "quant state: bad magic 0x%08x (not a qk_quant_state or corrupted)", st->magic);
    if (st->version != QK_STATE_VERSION)
        return fail(QK_ERR_BAD_STATE, "quant state: unknown version %u (this library reads %u)", st->version,
                    QK_STATE_VERSION);
    if (st->struct_bytes != sizeof(qk_quant_state))
        return fail(QK_ERR_BAD_STATE, "quant state: struct_bytes %u != %zu", st->struct_bytes, sizeof(qk_quant_state));
    if (st->rows < 1 || st->cols < 1 || st->n < 1)
        return fail(QK_ERR_BAD_STATE, "quant state: rows, cols and n must be >= 1");
    int64_t rc = 0;
    if (st->rows > (int64_t)1 << 40 || st->cols > (int64_t)1 << 40 || st->n > (int64_t)1 << 40 ||
        __builtin_mul_overflow(st->rows, st->cols, &rc) || st->n != rc)
        return fail(QK_ERR_BAD_STATE, "quant state: n (%lld) != rows (%lld) * cols (%lld)", (long long)st->n,
                    (long long)st->rows, (long long)st->cols);
    if (!valid_blocksize(st->blocksize))
        return fail(QK_ERR_BAD_STATE, "quant state: block size %d (expected 64, 128 or 256)", st->blocksize);
    if (st->codebook_kind < QK_NF4 || st->codebook_kind > QK_CUSTOM)
        return fail(QK_ERR_BAD_STATE, "quant state: unknown codebook kind %d", st->codebook_kind);
    if (st->reserved != 0) return fail(QK_ERR_BAD_STATE, "quant state: reserved field is not 0");
    for (int i = 0; i < 16; ++i)
        if (!std::isfinite(st->levels[i])) return fail(QK_ERR_BAD_STATE, "quant state: level %d is not finite", i);
    if (!st->codes) return fail(QK_ERR_BAD_STATE, "quant state: codes pointer is NULL");
    if (!aligned(st->codes, 4)) return fail(QK_ERR_BAD_STATE, "quant state: codes must be 4-byte aligned");
    if (st->nested == 1) {
        if (st->dq_blocksize != QK_DQ_BLOCK)
            return fail(QK_ERR_BAD_STATE, "quant state: nested with dq_blocksize %d (expected 256)", st->dq_blocksize);
        if (!st->q8 || !st->dq_scale || !st->dq_mean)
            return fail(QK_ERR_BAD_STATE, "quant state: nested needs q8, dq_scale and dq_mean");
        if (st->absmax) return fail(QK_ERR_BAD_STATE, "quant state: nested state also carries plain absmax");
        if (!aligned(st->dq_scale, 4) || !aligned(st->dq_mean, 4))
            return fail(QK_ERR_BAD_STATE, "quant state: dq_scale and dq_mean must be 4-byte aligned");
    } else if (st->nested == 0) {
        if (!st->absmax) return fail(QK_ERR_BAD_STATE, "quant state: plain state needs absmax");
        if (st->q8 || st->dq_scale || st->dq_mean || st->dq_blocksize != 0)
            return fail(QK_ERR_BAD_STATE, "quant state: plain state carries double-quant fields");
        if (!aligned(st->absmax, 4)) return fail(QK_ERR_BAD_STATE, "quant state: absmax must be 4-byte aligned");
    } else {
        return fail(QK_ERR_BAD_STATE, "quant state: nested flag %d (expected 0 or 1)", st->nested);
    }
    return QK_OK;
}

qk::DeqArgs deq_args(const qk_quant_state* st) {
    qk::DeqArgs a;
    a.codes = st->codes;
    a.absmax = st->absmax;
    a.q8 = st->q8;
    a.dq_scale = st->dq_scale;
    a.dq_mean = st->dq_mean;
    a.n = st->n;
    a.blocksize = st->blocksize;
    a.blocksize_log2 = st->blocksize == 64 ? 6 : st->blocksize == 128 ? 7 : 8;
    a.nested = st->nested;
    std::memcpy(a.levels, st->levels, sizeof(a.levels));
    return a;
}

thread_local const char* g_gemv_variant = "none";
thread_local const char* g_gemm_variant = "none";

}  // namespace

extern "C" {

qk_status qk_make_codebook(int32_t kind, float* levels_out) {
    if (!levels_out) return fail(QK_ERR_INVALID_ARG, "qk_make_codebook: levels_out is NULL");
    if (kind == QK_NF4) return qk::make_nf4(levels_out) == QK_OK ? ok() : QK_ERR_INVALID_ARG;
    if (kind == QK_FP4) return qk::make_fp4(levels_out) == QK_OK ? ok() : QK_ERR_INVALID_ARG;
    return fail(QK_ERR_INVALID_ARG, "qk_make_codebook: unknown kind %d (QK_NF4=0, QK_FP4=1)", kind);
}

qk_status qk_quantize_blockwise(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize, const float* levels,
                                uint8_t* codes, float* absmax, void* stream) {
    if (!x || !levels || !codes || !absmax)
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise: NULL pointer argument");
    if (n < 1 || n > ((int64_t)1 << 40))
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise: n must be in 1..2^40 (got %lld)", (long long)n);
    if (x_dtype != QK_BF16 && x_dtype != QK_F16 && x_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise: unknown x dtype %d", x_dtype);
    if (!valid_blocksize(blocksize))
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise: block size %d (expected 64, 128 or 256)", blocksize);
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(absmax, 4))
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise: x must be 16-byte aligned, codes and absmax 4-byte");
    qk::QuantLut lut;
    const char* why = "";
    const qk_status lst = qk::build_quant_lut(levels, &lut, &why);
    if (lst != QK_OK) return fail(lst, "qk_quantize_blockwise: %s", why);
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_quantize(x, x_dtype, n, blocksize, lut, codes, absmax,
                                        reinterpret_cast<hipStream_t>(stream)),
                    "qk_quantize_blockwise");
}

qk_status qk_quantize_blockwise_grouped(const qk_quant_task* tasks, int32_t ntasks, int32_t x_dtype,
                                        int32_t blocksize, const float* levels, void* stream) {
    const char* who = "qk_quantize_blockwise_grouped";
    if (!tasks || !levels) return fail(QK_ERR_INVALID_ARG, "%s: NULL tasks or levels", who);
    if (ntasks < 1 || ntasks > 256) return fail(QK_ERR_INVALID_ARG, "%s: ntasks must be in 1..256 (got %d)", who, ntasks);
    if (x_dtype != QK_BF16 && x_dtype != QK_F16 && x_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "%s: unknown x dtype %d", who, x_dtype);
    if (!valid_blocksize(blocksize))
        return fail(QK_ERR_INVALID_ARG, "%s: block size %d (expected 64, 128 or 256)", who, blocksize);
    const uintptr_t esize = x_dtype == QK_F32 ? 4 : 2;
    struct Span {
        uintptr_t lo, hi;
        bool out;
        int32_t task;
    };
    std::vector<Span> spans;
    std::vector<qk::QuantItem> items((size_t)ntasks);
    for (int32_t i = 0; i < ntasks; ++i) {
        const qk_quant_task& t = tasks[i];
        if (!t.x || !t.codes || !t.absmax) return fail(QK_ERR_INVALID_ARG, "%s: task %d: NULL pointer argument", who, i);
        if (t.n < 1 || t.n > ((int64_t)1 << 40))
            return fail(QK_ERR_INVALID_ARG, "%s: task %d: n must be in 1..2^40 (got %lld)", who, i, (long long)t.n);
        if (!aligned(t.x, 16) || !aligned(t.codes, 4) || !aligned(t.absmax, 4))
            return fail(QK_ERR_INVALID_ARG, "%s: task %d: x must be 16-byte aligned, codes and absmax 4-byte", who, i);
        const uintptr_t n = (uintptr_t)t.n;
        const uintptr_t nb = (n + (uintptr_t)blocksize - 1) / (uintptr_t)blocksize;
        spans.push_back({reinterpret_cast<uintptr_t>(t.x), reinterpret_cast<uintptr_t>(t.x) + esize * n, false, i});
        spans.push_back({reinterpret_cast<uintptr_t>(t.codes), reinterpret_cast<uintptr_t>(t.codes) + (n + 1) / 2, true, i});
        spans.push_back({reinterpret_cast<uintptr_t>(t.absmax), reinterpret_cast<uintptr_t>(t.absmax) + 4 * nb, true, i});
        items[(size_t)i] = qk::QuantItem{t.x, t.n, t.codes, t.absmax};
    }
    for (size_t a = 0; a < spans.size(); ++a) {
        if (!spans[a].out) continue;
        for (size_t b = 0; b < spans.size(); ++b) {
            if (a == b) continue;
            if (spans[a].lo < spans[b].hi && spans[b].lo < spans[a].hi)
                return fail(QK_ERR_INVALID_ARG, "%s: an output of task %d overlaps %s of task %d", who, spans[a].task,
                            spans[b].out ? "an output" : "the input", spans[b].task);
        }
    }
    qk::QuantLut lut;
    const char* why = "";
    const qk_status lst = qk::build_quant_lut(levels, &lut, &why);
    if (lst != QK_OK) return fail(lst, "%s: %s", who, why);
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_quantize_group(items.data(), ntasks, x_dtype, blocksize, lut,
                                              reinterpret_cast<hipStream_t>(stream)),
                    who);
}

qk_status qk_make_dynamic_map(int32_t is_signed, float* levels_out) {
    if (!levels_out) return fail(QK_ERR_INVALID_ARG, "qk_make_dynamic_map: levels_out is NULL");
    qk::make_dynamic_map(is_signed != 0 ? 1 : 0, levels_out);
    return ok();
}

namespace {
bool valid_blocksize8(int32_t b) { return b == 256 || b == 512 || b == 1024 || b == 2048 || b == 4096; }
}  // namespace

qk_status qk_quantize_blockwise_8bit(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize,
                                     const float* levels, uint8_t* codes, float* absmax, void* stream) {
    if (!x || !levels || !codes || !absmax)
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise_8bit: NULL pointer argument");
    if (n < 1) return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise_8bit: n must be >= 1 (got %lld)", (long long)n);
    if (x_dtype != QK_BF16 && x_dtype != QK_F16 && x_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise_8bit: unknown x dtype %d", x_dtype);
    if (!valid_blocksize8(blocksize))
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise_8bit: block size %d (expected 256, 512, 1024, 2048 or 4096)",
                    blocksize);
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(absmax, 4))
        return fail(QK_ERR_INVALID_ARG, "qk_quantize_blockwise_8bit: x must be 16-byte aligned, codes 8-byte, absmax 4-byte");
    qk::QuantLut8 lut;
    const char* why = "";
    const qk_status lst = qk::build_quant_lut8(levels, &lut, &why);
    if (lst != QK_OK) return fail(lst, "qk_quantize_blockwise_8bit: %s", why);
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_quantize8(x, x_dtype, n, blocksize, lut, codes, absmax,
                                         reinterpret_cast<hipStream_t>(stream)),
                    "qk_quantize_blockwise_8bit");
}

qk_status qk_dequantize_blockwise_8bit(const uint8_t* codes, const float* absmax, int64_t n, int32_t blocksize,
                                       const float* levels, void* out, int32_t out_dtype, void* stream) {
    if (!codes || !absmax || !levels || !out)
        return fail(QK_ERR_INVALID_ARG, "qk_dequantize_blockwise_8bit: NULL pointer argument");
    if (n < 1) return fail(QK_ERR_INVALID_ARG, "qk_dequantize_blockwise_8bit: n must be >= 1 (got %lld)", (long long)n);
    if (!valid_blocksize8(blocksize))
        return fail(QK_ERR_INVALID_ARG, "qk_dequantize_blockwise_8bit: block size %d (expected 256, 512, 1024, 2048 or 4096)",
                    blocksize);
    if (out_dtype != QK_F32 && out_dtype != QK_BF16)
        return fail(QK_ERR_INVALID_ARG, "qk_dequantize_blockwise_8bit: out dtype %d (expected QK_F32 or QK_BF16)", out_dtype);
    for (int i = 0; i < 256; ++i)
        if (!std::isfinite(levels[i]))
            return fail(QK_ERR_INVALID_ARG, "qk_dequantize_blockwise_8bit: levels[%d] is not finite", i);
    if (!aligned(codes, 8) || !aligned(absmax, 4) || !aligned(out, 16))
        return fail(QK_ERR_INVALID_ARG, "qk_dequantize_blockwise_8bit: codes must be 8-byte aligned, out 16-byte, absmax 4-byte");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_dequantize8(codes, absmax, n, blocksize, levels, out, out_dtype,
                                           reinterpret_cast<hipStream_t>(stream)),
                    "qk_dequantize_blockwise_8bit");
}

qk_status qk_int8_quantize_rows(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, const uint8_t* skip_cols,
                                int8_t* q, float* absmax, void* stream) {
    if (!x || !q || !absmax) return fail(QK_ERR_INVALID_ARG, "qk_int8_quantize_rows: NULL pointer argument");
    if (x_dtype != QK_BF16 && x_dtype != QK_F16 && x_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_quantize_rows: unknown x dtype %d", x_dtype);
    if (rows < 1 || cols < 1 || cols % 8 != 0)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_quantize_rows: rows >= 1 and cols >= 1 with cols %% 8 == 0");
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(absmax, 4) || (skip_cols && !aligned(skip_cols, 8)))
        return fail(QK_ERR_INVALID_ARG, "qk_int8_quantize_rows: x must be 16-byte aligned, q and skip_cols 8-byte");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_int8_rowquant(x, x_dtype, rows, cols, skip_cols, q, absmax,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "qk_int8_quantize_rows");
}

qk_status qk_int8_outlier_columns(const void* x, int32_t x_dtype, int64_t M, int64_t K, float threshold, float* colmax,
                                  uint8_t* flags, int32_t* idx, int32_t* count, void* stream) {
    if (!x || !colmax || !flags || !idx || !count)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_outlier_columns: NULL pointer argument");
    if (x_dtype != QK_BF16 && x_dtype != QK_F16 && x_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_outlier_columns: unknown x dtype %d", x_dtype);
    if (M < 1 || K < 1 || K % 8 != 0)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_outlier_columns: M >= 1 and K >= 1 with K %% 8 == 0");
    if (!std::isfinite(threshold) || threshold < 0.0f)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_outlier_columns: threshold must be finite and >= 0");
    if (!aligned(x, 16) || !aligned(colmax, 4) || !aligned(idx, 4) || !aligned(count, 4))
        return fail(QK_ERR_INVALID_ARG, "qk_int8_outlier_columns: x must be 16-byte aligned, colmax, idx, count 4-byte");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_int8_outliers(x, x_dtype, M, K, threshold, colmax, flags, idx, count,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "qk_int8_outlier_columns");
}

qk_status qk_int8_matmul(const int8_t* Xq, const float* SX, const int8_t* CB, const float* SCB, int64_t M, int64_t N,
                         int64_t K, const void* X, const int32_t* outlier_idx, const int32_t* outlier_count, void* Y,
                         void* stream) {
    if (!Xq || !SX || !CB || !SCB || !Y) return fail(QK_ERR_INVALID_ARG, "qk_int8_matmul: NULL pointer argument");
    const bool any = X || outlier_idx || outlier_count;
    if (any && !(X && outlier_idx && outlier_count))
        return fail(QK_ERR_INVALID_ARG, "qk_int8_matmul: give X, outlier_idx and outlier_count together, or none");
    if (M < 1 || N < 1 || K < 16 || K % 16 != 0)
        return fail(QK_ERR_INVALID_ARG, "qk_int8_matmul: M, N >= 1 and K >= 16 with K %% 16 == 0");
    if (!aligned(Xq, 16) || !aligned(CB, 16) || !aligned(SX, 4) || !aligned(SCB, 4) || !aligned(Y, 2) ||
        (any && (!aligned(X, 2) || !aligned(outlier_idx, 4) || !aligned(outlier_count, 4))))
        return fail(QK_ERR_INVALID_ARG, "qk_int8_matmul: Xq and CB must be 16-byte aligned, the others element-aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_int8_matmul(Xq, SX, CB, SCB, M, N, K, X, outlier_idx, outlier_count, Y,
                                           reinterpret_cast<hipStream_t>(stream)),
                    "qk_int8_matmul");
}

qk_status qk_double_quant_workspace_size(int64_t nblocks, size_t* bytes) {
    if (!bytes) return fail(QK_ERR_INVALID_ARG, "qk_double_quant_workspace_size: bytes is NULL");
    if (nblocks < 1) return fail(QK_ERR_INVALID_ARG, "qk_double_quant_workspace_size: nblocks must be >= 1");
    *bytes = qk::dq_workspace_bytes(nblocks);
    return ok();
}

qk_status qk_double_quant(const float* absmax, int64_t nblocks, int32_t dq_blocksize, int8_t* q8, float* scale,
                          float* mean, void* workspace, size_t workspace_bytes, void* stream) {
    if (!absmax || !q8 || !scale || !mean) return fail(QK_ERR_INVALID_ARG, "qk_double_quant: NULL pointer argument");
    if (nblocks < 1) return fail(QK_ERR_INVALID_ARG, "qk_double_quant: nblocks must be >= 1");
    if (dq_blocksize != QK_DQ_BLOCK)
        return fail(QK_ERR_UNSUPPORTED, "qk_double_quant: dq_blocksize %d (only 256 is implemented)", dq_blocksize);
    if (!aligned(absmax, 4) || !aligned(q8, 4) || !aligned(scale, 4) || !aligned(mean, 4))
        return fail(QK_ERR_INVALID_ARG, "qk_double_quant: absmax, q8, scale and mean must be 4-byte aligned");
    const size_t need = qk::dq_workspace_bytes(nblocks);
    if (!workspace || workspace_bytes < need)
        return fail(QK_ERR_WORKSPACE, "qk_double_quant: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 8)) return fail(QK_ERR_INVALID_ARG, "qk_double_quant: workspace must be 8-byte aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_double_quant(absmax, nblocks, q8, scale, mean, workspace,
                                            reinterpret_cast<hipStream_t>(stream)),
                    "qk_double_quant");
}

namespace {

// the grouped double quantization's arguments (no device access): sizes, pointers,
// alignment, and that no output overlaps another output or an input
qk_status check_dq_tasks(const qk_dq_task* tasks, int32_t ntasks, const char* who) {
    if (!tasks) return fail(QK_ERR_INVALID_ARG, "%s: tasks is NULL", who);
    if (ntasks < 1 || ntasks > 256) return fail(QK_ERR_INVALID_ARG, "%s: ntasks must be in 1..256 (got %d)", who, ntasks);
    struct Span {
        uintptr_t lo, hi;
        bool out;
        int32_t task;
    };
    std::vector<Span> spans;
    for (int32_t i = 0; i < ntasks; ++i) {
        const qk_dq_task& t = tasks[i];
        if (t.nblocks < 1) return fail(QK_ERR_INVALID_ARG, "%s: task %d: nblocks must be >= 1", who, i);
        if (!t.absmax || !t.q8 || !t.scale || !t.mean)
            return fail(QK_ERR_INVALID_ARG, "%s: task %d: NULL pointer argument", who, i);
        if (!aligned(t.absmax, 4) || !aligned(t.q8, 4) || !aligned(t.scale, 4) || !aligned(t.mean, 4))
            return fail(QK_ERR_INVALID_ARG, "%s: task %d: absmax, q8, scale and mean must be 4-byte aligned", who, i);
        const uintptr_t nb = (uintptr_t)t.nblocks;
        const uintptr_t nd = (nb + QK_DQ_BLOCK - 1) / QK_DQ_BLOCK;
        spans.push_back({reinterpret_cast<uintptr_t>(t.absmax), reinterpret_cast<uintptr_t>(t.absmax) + 4 * nb, false, i});
        spans.push_back({reinterpret_cast<uintptr_t>(t.q8), reinterpret_cast<uintptr_t>(t.q8) + nb, true, i});
        spans.push_back({reinterpret_cast<uintptr_t>(t.scale), reinterpret_cast<uintptr_t>(t.scale) + 4 * nd, true, i});
        spans.push_back({reinterpret_cast<uintptr_t>(t.mean), reinterpret_cast<uintptr_t>(t.mean) + 4, true, i});
    }
    for (size_t a = 0; a < spans.size(); ++a) {
        if (!spans[a].out) continue;
        for (size_t b = 0; b < spans.size(); ++b) {
            if (a == b) continue;
            if (spans[a].lo < spans[b].hi && spans[b].lo < spans[a].hi)
                return fail(QK_ERR_INVALID_ARG, "%s: an output of task %d overlaps %s of task %d", who, spans[a].task,
                            spans[b].out ? "an output" : "the absmax", spans[b].task);
        }
    }
    return ok();
}

size_t dq_group_workspace(const qk_dq_task* tasks, int32_t ntasks) {
    size_t total = 0;
    for (int32_t i = 0; i < ntasks; ++i) total += qk::dq_workspace_bytes(tasks[i].nblocks);
    return total;
}

}  // namespace

qk_status qk_double_quant_grouped_workspace_size(const qk_dq_task* tasks, int32_t ntasks, size_t* bytes) {
    if (!bytes) return fail(QK_ERR_INVALID_ARG, "qk_double_quant_grouped_workspace_size: bytes is NULL");
    if (!tasks) return fail(QK_ERR_INVALID_ARG, "qk_double_quant_grouped_workspace_size: tasks is NULL");
    if (ntasks < 1 || ntasks > 256)
        return fail(QK_ERR_INVALID_ARG, "qk_double_quant_grouped_workspace_size: ntasks must be in 1..256 (got %d)",
                    ntasks);
    for (int32_t i = 0; i < ntasks; ++i)
        if (tasks[i].nblocks < 1)
            return fail(QK_ERR_INVALID_ARG, "qk_double_quant_grouped_workspace_size: task %d: nblocks must be >= 1", i);
    *bytes = dq_group_workspace(tasks, ntasks);
    return ok();
}

qk_status qk_double_quant_grouped(const qk_dq_task* tasks, int32_t ntasks, int32_t dq_blocksize, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    const qk_status v = check_dq_tasks(tasks, ntasks, "qk_double_quant_grouped");
    if (v != QK_OK) return v;
    if (dq_blocksize != QK_DQ_BLOCK)
        return fail(QK_ERR_UNSUPPORTED, "qk_double_quant_grouped: dq_blocksize %d (only 256 is implemented)", dq_blocksize);
    const size_t need = dq_group_workspace(tasks, ntasks);
    if (!workspace || workspace_bytes < need)
        return fail(QK_ERR_WORKSPACE, "qk_double_quant_grouped: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 8))
        return fail(QK_ERR_INVALID_ARG, "qk_double_quant_grouped: workspace must be 8-byte aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    std::vector<qk::DqItem> items((size_t)ntasks);
    for (int32_t i = 0; i < ntasks; ++i)
        items[(size_t)i] = qk::DqItem{tasks[i].absmax, tasks[i].nblocks, tasks[i].q8, tasks[i].scale, tasks[i].mean};
    return launched(qk::launch_double_quant_group(items.data(), ntasks, workspace, reinterpret_cast<hipStream_t>(stream)),
                    "qk_double_quant_grouped");
}

qk_status qk_state_init(qk_quant_state* st, int32_t codebook_kind, const float* levels, int64_t rows, int64_t cols,
                        int32_t blocksize, const uint8_t* codes, const float* absmax, const int8_t* q8,
                        const float* dq_scale, const float* dq_mean) {
    if (!st || !levels || !codes) return fail(QK_ERR_INVALID_ARG, "qk_state_init: NULL state, levels or codes");
    if (rows < 1 || cols < 1) return fail(QK_ERR_INVALID_ARG, "qk_state_init: rows and cols must be >= 1");
    if (!valid_blocksize(blocksize))
        return fail(QK_ERR_INVALID_ARG, "qk_state_init: block size %d (expected 64, 128 or 256)", blocksize);
    const bool nested = q8 || dq_scale || dq_mean;
    if (nested && absmax) return fail(QK_ERR_INVALID_ARG, "qk_state_init: give either absmax or q8/dq_scale/dq_mean");
    if (nested && !(q8 && dq_scale && dq_mean))
        return fail(QK_ERR_INVALID_ARG, "qk_state_init: a nested state needs q8, dq_scale and dq_mean");
    if (!nested && !absmax) return fail(QK_ERR_INVALID_ARG, "qk_state_init: absmax is NULL");
    std::memset(st, 0, sizeof(*st));
    st->magic = QK_STATE_MAGIC;
    st->version = QK_STATE_VERSION;
    st->struct_bytes = sizeof(qk_quant_state);
    st->codebook_kind = codebook_kind;
    st->rows = rows;
    st->cols = cols;
    st->n = rows * cols;
    st->blocksize = blocksize;
    st->nested = nested ? 1 : 0;
    st->dq_blocksize = nested ? QK_DQ_BLOCK : 0;
    std::memcpy(st->levels, levels, sizeof(st->levels));
    st->codes = codes;
    st->absmax = absmax;
    st->q8 = q8;
    st->dq_scale = dq_scale;
    st->dq_mean = dq_mean;
    return ok();
}

qk_status qk_dequantize(const qk_quant_state* st, void* out, int32_t out_dtype, void* stream) {
    const qk_status v = validate_state(st);
    if (v != QK_OK) return v;
    if (!out) return fail(QK_ERR_INVALID_ARG, "qk_dequantize: out is NULL");
    if (out_dtype != QK_BF16 && out_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "qk_dequantize: out dtype %d (expected QK_F32 or QK_BF16)", out_dtype);
    if (!aligned(out, 16)) return fail(QK_ERR_INVALID_ARG, "qk_dequantize: out must be 16-byte aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_dequantize(deq_args(st), out, out_dtype, reinterpret_cast<hipStream_t>(stream)),
                    "qk_dequantize");
}

qk_status qk_dequantize_grouped(const qk_dequant_task* tasks, int32_t ntasks, int32_t out_dtype, void* stream) {
    const char* who = "qk_dequantize_grouped";
    if (!tasks) return fail(QK_ERR_INVALID_ARG, "%s: tasks is NULL", who);
    if (ntasks < 1 || ntasks > 256) return fail(QK_ERR_INVALID_ARG, "%s: ntasks must be in 1..256 (got %d)", who, ntasks);
    if (out_dtype != QK_BF16 && out_dtype != QK_F32)
        return fail(QK_ERR_INVALID_ARG, "%s: out dtype %d (expected QK_F32 or QK_BF16)", who, out_dtype);
    const uintptr_t esize = out_dtype == QK_BF16 ? 2 : 4;
    std::vector<qk::DeqItem> items((size_t)ntasks);
    for (int32_t i = 0; i < ntasks; ++i) {
        const qk_status v = validate_state(tasks[i].st);
        if (v != QK_OK) return v;
        if (!tasks[i].out) return fail(QK_ERR_INVALID_ARG, "%s: task %d: out is NULL", who, i);
        if (!aligned(tasks[i].out, 16)) return fail(QK_ERR_INVALID_ARG, "%s: task %d: out must be 16-byte aligned", who, i);
        items[i] = qk::DeqItem{deq_args(tasks[i].st), tasks[i].out};
    }
    // the arrays of a launch are written at once: every out must be disjoint from the others
    for (int32_t i = 0; i < ntasks; ++i) {
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(tasks[i].out);
        const uintptr_t o1 = o0 + (uintptr_t)tasks[i].st->n * esize;
        for (int32_t j = i + 1; j < ntasks; ++j) {
            const uintptr_t p0 = reinterpret_cast<uintptr_t>(tasks[j].out);
            const uintptr_t p1 = p0 + (uintptr_t)tasks[j].st->n * esize;
            if (p0 < o1 && o0 < p1) return fail(QK_ERR_INVALID_ARG, "%s: out of task %d overlaps out of task %d", who, i, j);
        }
    }
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_dequantize_group(items.data(), ntasks, out_dtype, reinterpret_cast<hipStream_t>(stream)),
                    who);
}

qk_status qk_lora_merge(const qk_quant_state* st, const void* A, const void* B, int32_t r, float lora_scale,
                        void* out, void* stream) {
    const qk_status v = validate_state(st);
    if (v != QK_OK) return v;
    if (!A || !B || !out) return fail(QK_ERR_INVALID_ARG, "qk_lora_merge: NULL A, B or out");
    if (r < 1 || r > 1024) return fail(QK_ERR_INVALID_ARG, "qk_lora_merge: rank must be in 1..1024 (got %d)", r);
    if (!std::isfinite(lora_scale)) return fail(QK_ERR_INVALID_ARG, "qk_lora_merge: lora_scale is not finite");
    if (!aligned(A, 2) || !aligned(B, 2) || !aligned(out, 2))
        return fail(QK_ERR_INVALID_ARG, "qk_lora_merge: bf16 buffers must be 2-byte aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    qk::MatArgs w{deq_args(st), st->rows, st->cols};
    return launched(qk::launch_lora_merge(w, A, B, r, lora_scale, out, reinterpret_cast<hipStream_t>(stream)),
                    "qk_lora_merge");
}

qk_status qk_qlora_backward_workspace_size(int64_t M, const qk_quant_state* st, int32_t r, size_t* bytes) {
    if (!bytes) return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward_workspace_size: bytes is NULL");
    const qk_status v = validate_state(st);
    if (v != QK_OK) return v;
    if (M < 1 || r < 0 || r > 64)
        return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward_workspace_size: M >= 1, r in 0..64");
    *bytes = qk::qlora_backward_workspace_bytes(M, st->rows, st->cols, r);
    return ok();
}

qk_status qk_qlora_backward(const void* dY, int64_t M, const qk_quant_state* st, const void* X, const void* A,
                            const void* B, int32_t r, float lora_scale, void* dX, float* dA, float* dB,
                            void* workspace, size_t workspace_bytes, void* stream) {
    const qk_status v = validate_state(st);
    if (v != QK_OK) return v;
    if (!dY || !dX) return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: NULL dY or dX");
    if (M < 1 || M > 65535LL * 128) return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: M must be in 1..8388480");
    if ((A == nullptr) != (B == nullptr))
        return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: give both LoRA A and B, or neither");
    const bool lora = A != nullptr;
    if (lora && (r < 1 || r > 64)) return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: LoRA rank must be in 1..64");
    if (lora && (!X || !dA || !dB)) return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: LoRA needs X, dA and dB");
    if (lora && !std::isfinite(lora_scale)) return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: lora_scale is not finite");
    if (st->rows % 64 != 0 || st->cols % 64 != 0)
        return fail(QK_ERR_UNSUPPORTED, "qk_qlora_backward: W [%lld, %lld] needs both sizes multiples of 64",
                    (long long)st->rows, (long long)st->cols);
    if (!aligned(dY, 16) || !aligned(dX, 2) || (lora && (!aligned(X, 16) || !aligned(A, 2) || !aligned(B, 2) ||
                                                         !aligned(dA, 4) || !aligned(dB, 4))))
        return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: dY and X must be 16-byte aligned, the others element-aligned");
    const size_t need = qk::qlora_backward_workspace_bytes(M, st->rows, st->cols, lora ? r : 0);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QK_ERR_WORKSPACE, "qk_qlora_backward: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned(workspace, 16))
        return fail(QK_ERR_INVALID_ARG, "qk_qlora_backward: workspace must be 16-byte aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    qk::MatArgs w{deq_args(st), st->rows, st->cols};
    return launched(qk::launch_qlora_backward(dY, M, w, X, A, B, lora ? r : 0, lora_scale, dX, dA, dB, workspace,
                                              reinterpret_cast<hipStream_t>(stream)),
                    "qk_qlora_backward");
}

qk_status qk_gemv_nf4_grouped(const qk_gemv_task* tasks, int32_t ntasks, int32_t M, void* stream) {
    if (!tasks) return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: tasks is NULL");
    if (ntasks < 1 || ntasks > 256)
        return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: ntasks must be in 1..256 (got %d)", ntasks);
    if (M < 1 || M > 16) return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: M must be in 1..16 (got %d)", M);
    std::vector<qk::GemvItem> items((size_t)ntasks);
    for (int32_t i = 0; i < ntasks; ++i) {
        const qk_gemv_task& t = tasks[i];
        const qk_status v = validate_state(t.st);
        if (v != QK_OK) return v;
        if (!t.x || !t.y) return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: task %d: NULL x or y", i);
        if (!aligned(t.x, 16) || !aligned(t.y, 2))
            return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: task %d: x must be 16-byte aligned, y 2-byte", i);
        items[i] = qk::GemvItem{t.x, t.y, qk::MatArgs{deq_args(t.st), t.st->rows, t.st->cols}};
    }
    // every y must be disjoint from the other ys and from every x
    for (int32_t i = 0; i < ntasks; ++i) {
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(tasks[i].y);
        const uintptr_t y1 = y0 + (uintptr_t)M * (uintptr_t)tasks[i].st->rows * 2;
        for (int32_t j = 0; j < ntasks; ++j) {
            const uintptr_t x0 = reinterpret_cast<uintptr_t>(tasks[j].x);
            const uintptr_t x1 = x0 + (uintptr_t)M * (uintptr_t)tasks[j].st->cols * 2;
            if (x0 < y1 && y0 < x1)
                return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: y of task %d overlaps x of task %d", i, j);
            if (j == i) continue;
            const uintptr_t z0 = reinterpret_cast<uintptr_t>(tasks[j].y);
            const uintptr_t z1 = z0 + (uintptr_t)M * (uintptr_t)tasks[j].st->rows * 2;
            if (z0 < y1 && y0 < z1)
                return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4_grouped: y of task %d overlaps y of task %d", i, j);
        }
    }
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_gemv_group(items.data(), ntasks, M, reinterpret_cast<hipStream_t>(stream),
                                          &g_gemv_variant),
                    "qk_gemv_nf4_grouped");
}

qk_status qk_gemv_nf4(const void* x, int32_t M, const qk_quant_state* st, void* y, void* stream) {
    const qk_status v = validate_state(st);
    if (v != QK_OK) return v;
    if (!x || !y) return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4: NULL x or y");
    if (M < 1 || M > 16) return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4: M must be in 1..16 (got %d)", M);
    if (!aligned(x, 16) || !aligned(y, 2)) return fail(QK_ERR_INVALID_ARG, "qk_gemv_nf4: x must be 16-byte aligned, y 2-byte");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    qk::MatArgs w{deq_args(st), st->rows, st->cols};
    return launched(qk::launch_gemv(x, M, w, y, reinterpret_cast<hipStream_t>(stream), &g_gemv_variant),
                    "qk_gemv_nf4");
}

qk_status qk_gemm_nf4_workspace_size(int64_t M, int32_t r, size_t* bytes) {
    if (!bytes) return fail(QK_ERR_INVALID_ARG, "qk_gemm_nf4_workspace_size: bytes is NULL");
    if (M < 1 || r < 0 || r > 64) return fail(QK_ERR_INVALID_ARG, "qk_gemm_nf4_workspace_size: M >= 1, r in 0..64");
    *bytes = qk::gemm_workspace_bytes(M, r);
    return ok();
}

namespace {
qk_status check_gemm_args(const char* fn, const void* X, int64_t M, const qk_quant_state* st, const void* A,
                          const void* B, int32_t r, float lora_scale, const void* Y) {
    const qk_status v = validate_state(st);
    if (v != QK_OK) return v;
    if (!X || !Y) return fail(QK_ERR_INVALID_ARG, "%s: NULL X or Y", fn);
    if (M < 1 || M > ((int64_t)1 << 31)) return fail(QK_ERR_INVALID_ARG, "%s: M must be in 1..2^31", fn);
    if ((A == nullptr) != (B == nullptr)) return fail(QK_ERR_INVALID_ARG, "%s: give both LoRA A and B, or neither", fn);
    if (A && (r < 1 || r > 64)) return fail(QK_ERR_INVALID_ARG, "%s: LoRA rank must be in 1..64 (got %d)", fn, r);
    if (A && !std::isfinite(lora_scale)) return fail(QK_ERR_INVALID_ARG, "%s: lora_scale is not finite", fn);
    if (!aligned(X, 2) || !aligned(Y, 2) || (A && (!aligned(A, 2) || !aligned(B, 2))))
        return fail(QK_ERR_INVALID_ARG, "%s: bf16 buffers must be 2-byte aligned", fn);
    return QK_OK;
}
}  // namespace

qk_status qk_gemm_nf4(const void* X, int64_t M, const qk_quant_state* st, const void* A, const void* B, int32_t r,
                      float lora_scale, void* Y, void* workspace, size_t workspace_bytes, void* stream) {
    const qk_status v = check_gemm_args("qk_gemm_nf4", X, M, st, A, B, r, lora_scale, Y);
    if (v != QK_OK) return v;
    const size_t need = qk::gemm_workspace_bytes(M, A ? r : 0);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QK_ERR_WORKSPACE, "qk_gemm_nf4: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned(workspace, 16)) return fail(QK_ERR_INVALID_ARG, "qk_gemm_nf4: workspace must be 16-byte aligned");
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    qk::MatArgs w{deq_args(st), st->rows, st->cols};
    return launched(qk::launch_gemm(X, M, w, A, B, A ? r : 0, lora_scale, Y, workspace,
                                    reinterpret_cast<hipStream_t>(stream), &g_gemm_variant),
                    "qk_gemm_nf4");
}

namespace {
qk_status gemm_group_items(const char* who, const qk_gemm_task* tasks, int32_t ntasks, std::vector<qk::GemmItem>& items) {
    if (!tasks) return fail(QK_ERR_INVALID_ARG, "%s: tasks is NULL", who);
    if (ntasks < 1 || ntasks > 256) return fail(QK_ERR_INVALID_ARG, "%s: ntasks must be in 1..256 (got %d)", who, ntasks);
    items.resize((size_t)ntasks);
    for (int32_t i = 0; i < ntasks; ++i) {
        const qk_gemm_task& t = tasks[i];
        char fn[64];
        std::snprintf(fn, sizeof(fn), "%s: task %d", who, i);
        const qk_status v = check_gemm_args(fn, t.X, t.M, t.st, t.A, t.B, t.r, t.lora_scale, t.Y);
        if (v != QK_OK) return v;
        items[i] = qk::GemmItem{t.X, t.M, qk::MatArgs{deq_args(t.st), t.st->rows, t.st->cols}, t.A, t.B,
                                t.A ? t.r : 0, t.lora_scale, t.Y};
    }
    return QK_OK;
}
}  // namespace

qk_status qk_gemm_nf4_grouped_workspace_size(const qk_gemm_task* tasks, int32_t ntasks, size_t* bytes) {
    if (!bytes) return fail(QK_ERR_INVALID_ARG, "qk_gemm_nf4_grouped_workspace_size: bytes is NULL");
    std::vector<qk::GemmItem> items;
    const qk_status v = gemm_group_items("qk_gemm_nf4_grouped_workspace_size", tasks, ntasks, items);
    if (v != QK_OK) return v;
    *bytes = qk::gemm_group_workspace_bytes(items.data(), ntasks);
    return ok();
}

qk_status qk_gemm_nf4_grouped(const qk_gemm_task* tasks, int32_t ntasks, void* workspace, size_t workspace_bytes,
                              void* stream) {
    const char* who = "qk_gemm_nf4_grouped";
    std::vector<qk::GemmItem> items;
    const qk_status v = gemm_group_items(who, tasks, ntasks, items);
    if (v != QK_OK) return v;
    const size_t need = qk::gemm_group_workspace_bytes(items.data(), ntasks);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QK_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned(workspace, 16)) return fail(QK_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", who);
    // the GEMMs of a launch run at once: every Y must be disjoint from the other Ys, from
    // every X and from the workspace
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + need;
    for (int32_t i = 0; i < ntasks; ++i) {
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(tasks[i].Y);
        const uintptr_t y1 = y0 + (uintptr_t)tasks[i].M * (uintptr_t)tasks[i].st->rows * 2;
        if (need > 0 && w0 < y1 && y0 < w1)
            return fail(QK_ERR_INVALID_ARG, "%s: Y of task %d overlaps the workspace", who, i);
        for (int32_t j = 0; j < ntasks; ++j) {
            const uintptr_t x0 = reinterpret_cast<uintptr_t>(tasks[j].X);
            const uintptr_t x1 = x0 + (uintptr_t)tasks[j].M * (uintptr_t)tasks[j].st->cols * 2;
            if (x0 < y1 && y0 < x1) return fail(QK_ERR_INVALID_ARG, "%s: Y of task %d overlaps X of task %d", who, i, j);
            if (j == i) continue;
            const uintptr_t z0 = reinterpret_cast<uintptr_t>(tasks[j].Y);
            const uintptr_t z1 = z0 + (uintptr_t)tasks[j].M * (uintptr_t)tasks[j].st->rows * 2;
            if (z0 < y1 && y0 < z1) return fail(QK_ERR_INVALID_ARG, "%s: Y of task %d overlaps Y of task %d", who, i, j);
        }
    }
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    return launched(qk::launch_gemm_group(items.data(), ntasks, workspace, reinterpret_cast<hipStream_t>(stream),
                                          &g_gemm_variant),
                    who);
}

qk_status qk_gemm_nf4_noalloc(const void* X, int64_t M, const qk_quant_state* st, const void* A, const void* B,
                              int32_t r, float lora_scale, void* Y, void* stream) {
    const qk_status v = check_gemm_args("qk_gemm_nf4_noalloc", X, M, st, A, B, r, lora_scale, Y);
    if (v != QK_OK) return v;
    const size_t need = qk::gemm_workspace_bytes(M, A ? r : 0);
    const size_t cap = qk::gemm_noalloc_scratch_bytes();
    if (need > cap)
        return fail(QK_ERR_WORKSPACE,
                    "qk_gemm_nf4_noalloc: the LoRA partials of M = %lld, r = %d need %zu bytes; the static scratch "
                    "holds %zu (M * 16 * ceil(r / 16) <= %zu); use qk_gemm_nf4 with a workspace",
                    (long long)M, r, need, cap, cap / (8 * sizeof(float)));
    const qk_status dev = ensure_device();
    if (dev != QK_OK) return dev;
    void* scratch = nullptr;
    if (need > 0) {
        const hipError_t e = qk::gemm_noalloc_scratch(&scratch);
        if (e != hipSuccess)
            return fail(QK_ERR_HIP, "qk_gemm_nf4_noalloc: address of the static scratch: %s", hipGetErrorString(e));
    }
    qk::MatArgs w{deq_args(st), st->rows, st->cols};
    return launched(qk::launch_gemm(X, M, w, A, B, A ? r : 0, lora_scale, Y, scratch,
                                    reinterpret_cast<hipStream_t>(stream), &g_gemm_variant),
                    "qk_gemm_nf4_noalloc");
}

const char* qk_last_error(void) { return g_last_error.c_str(); }

const char* qk_version(void) { return "qk 0.1.0 gfx950"; }

const char* qk_backend_info(void) {
    static thread_local std::string s;
    s = std::string("quantize: wave per 512 elements, DPP block absmax, reciprocal+Markstein division, LDS bin table; ") +
        "double_quant: fp64 tree partials + int8 per 256; dequantize: LDS levels; gemv: " + g_gemv_variant +
        "; gemm: " + g_gemm_variant +
        "; lora_merge: fp32 adapter sum in LDS, fused dequant; qlora_backward: dX 256x128 tiles mfma 32x32x16 bf16 with "
        "W^T dequantized into LDS, dA/dB row-slice reductions; quantize_8bit: LDS bin table built per workgroup; "
        "int8_matmul: mfma 32x32x32 i8 256x256 tiles 8 waves, fp16 outlier mfma in the epilogue";
    return s.c_str();
}

}  // extern "C"
