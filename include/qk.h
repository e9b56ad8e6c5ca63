/*
 * qk.h — C ABI of a blockwise 4-bit weight quantization library for AMD MI355X
 * (gfx950): NF4 / FP4 quantize and dequantize with one fp32 absmax per block,
 * double quantization of the absmax array, and the dequantize-fused decode GEMV
 * and prefill / training GEMM of a frozen QLoRA base layer.
 *
 * Sources of the definitions (cited by page title and section):
 *  [NF4]   "篇2-bitsandbytes-具体观-算法与实现剖析" (xyzblog), §2.2 QLoRA / NF4,
 *          【原理】① (NF4 levels: 16 equal-probability slabs of N(0,1), each
 *          represented by its midpoint, normalised to [-1, 1]), 【原理】② (double
 *          quantization of the absmax), 【代码】 (quantize_4bit with blocksize 64,
 *          quant_type nf4 / fp4, compress_statistics; the quant_state fields
 *          absmax / code / state2 / offset / nested_absmax; FP4 built as the
 *          2-exponent-bit, 1-mantissa-bit signed case of a generic float-format
 *          table; the 4-bit linear forward = dequantize + matmul), 【例子】 and
 *          figure 2-2 (the pipeline: split into blocks of 64, absmax per block,
 *          divide, table lookup, pack two codes per byte, quantize the absmax
 *          again into state2).
 *  [DEQ]   "LLM 相關知識" (technicalnotes, tag qlora), section 5 動態反量化:
 *          the 4-bit base is restored to BF16 layer by layer right before its
 *          matmul; section 2-2 LoRA and section 8 (merge / no-merge): the
 *          layer output is the base output plus the LoRA output X·A·B.
 *  [OPT8]  "篇2-bitsandbytes-具体观-算法与实现剖析", §2.3 8-bit Optimizers,
 *          【原理】 and figure 2-3: optimizer states in blocks of 2048, one local
 *          absmax per block, 8-bit codes through a dynamic map of 256
 *          non-uniform levels (dense at zero, sparse in the tails, maximising the
 *          code entropy; signed "dynamic" and unsigned "udynamic" variants).
 *  [INT8]  "篇2-bitsandbytes-具体观-算法与实现剖析", §2.1 LLM.int8(), 【原理】,
 *          【代码】, 【例子】 and figure 2-1: activation columns whose largest
 *          magnitude exceeds a threshold go through a 16-bit matmul with the
 *          matching weight columns; the rest is quantized vector-wise (one absmax
 *          per row, scaled to [-127, 127], int8) and multiplied with the int8
 *          weight (CB, with one absmax per weight row SCB); the results are added;
 *          threshold 0 disables the decomposition.
 *  [YOLO]  "Tim Dettmers 如何用 bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？"
 *          (yololab), sections on NF4, double quantization and QLoRA: the
 *          quantizer, loader and kernel must share exactly one definition of
 *          codebook, block size, scale and packing.
 *
 * Conventions for every call
 *  - Memory: the caller owns every buffer.  Pointers documented "device" must
 *    point to device memory of the current HIP device; "host" pointers to
 *    ordinary host memory.  The library allocates no device memory and frees
 *    nothing; calls that need scratch space take a caller workspace whose size
 *    a *_workspace_size query returns.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Every device call is asynchronous on that stream and never
 *    synchronizes.
 *  - Errors: every call returns a qk_status.  Arguments are validated on the
 *    host before anything is launched, and no device pointer is dereferenced on
 *    the host; a rejected call launches nothing.  A message for the last
 *    failure of the calling thread is available from qk_last_error().
 *  - Numerics: inputs must be finite (not checked in the kernels).  All sizes
 *    are element counts unless stated otherwise.
 *  - Layout of a quantized tensor of n elements, block size B (the weight
 *    W[N, K] is row-major, so n = N*K and blocks run over the flattened
 *    tensor; a block may straddle two rows when K % B != 0):
 *      codes     uint8  [ceil(n/2)]  element 2t in the high nibble of byte t,
 *                                    element 2t+1 in the low nibble; the low
 *                                    nibble of the last byte is 0 when n is odd
 *      absmax    fp32   [nb]         nb = ceil(n/B), block j = [jB, min(jB+B, n))
 *      or, double-quantized (nested):
 *      q8        int8   [nb]
 *      dq_scale  fp32   [nd]         nd = ceil(nb/256)
 *      dq_mean   fp32   [1]
 */
#ifndef QK_H
#define QK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qk_status;
enum {
    QK_OK = 0,
    QK_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad enum, misaligned buffer */
    QK_ERR_UNSUPPORTED = -2,   /* valid request the library does not implement */
    QK_ERR_BAD_STATE = -3,     /* qk_quant_state with a wrong magic, version, size or
                                  inconsistent fields (unknown or corrupted metadata) */
    QK_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed */
    QK_ERR_NO_DEVICE = -5,     /* no usable gfx950 device */
    QK_ERR_WORKSPACE = -6      /* workspace missing or smaller than required */
};

/* element types */
enum { QK_F32 = 0, QK_BF16 = 1, QK_F16 = 2 };

/* level tables */
enum { QK_NF4 = 0, QK_FP4 = 1, QK_CUSTOM = 2 };

#define QK_STATE_MAGIC 0x314B5451u   /* "QTK1" little-endian */
#define QK_STATE_VERSION 1u
#define QK_DQ_BLOCK 256

/*
 * Descriptor of one quantized tensor (the [NF4] quant_state).  Plain data: the
 * pointers are device pointers owned by the caller.  Build it with
 * qk_state_init(); a descriptor whose magic, version or struct_bytes do not
 * match, or whose fields disagree (n != rows*cols, bad block size, missing
 * pointers), is rejected with QK_ERR_BAD_STATE by every call that takes one.
 */
typedef struct qk_quant_state {
    uint32_t magic;          /* QK_STATE_MAGIC */
    uint32_t version;        /* QK_STATE_VERSION */
    uint32_t struct_bytes;   /* sizeof(qk_quant_state) */
    int32_t codebook_kind;   /* QK_NF4, QK_FP4 or QK_CUSTOM (informative) */
    int64_t n;               /* number of elements = rows * cols */
    int64_t rows;            /* N: output features of the weight */
    int64_t cols;            /* K: input features of the weight */
    int32_t blocksize;       /* B: 64, 128 or 256 */
    int32_t nested;          /* 1: absmax is double-quantized (q8, dq_scale, dq_mean) */
    int32_t dq_blocksize;    /* 256 when nested, else 0 */
    int32_t reserved;        /* 0 */
    float levels[16];        /* level of each 4-bit code, in code order */
    const uint8_t* codes;    /* device, [ceil(n/2)], 4-byte aligned */
    const float* absmax;     /* device, [nb], when !nested (else NULL) */
    const int8_t* q8;        /* device, [nb], when nested (else NULL) */
    const float* dq_scale;   /* device, [ceil(nb/256)], when nested (else NULL) */
    const float* dq_mean;    /* device, [1], when nested (else NULL) */
} qk_quant_state;

/*
 * qk_make_codebook — host.  [NF4] 【原理】① and 【代码】.
 *   kind QK_NF4: levels[i] = RN_fp32( Phi^-1((2i+1)/32) / Phi^-1(31/32) ),
 *       i = 0..15, with Phi^-1 the standard normal quantile evaluated in fp64
 *       (Wichura's algorithm AS 241); symmetric, strictly increasing, no zero.
 *   kind QK_FP4: the signed E2M1 minifloat with subnormals in code order
 *       (code = sign<<3 | exponent<<1 | mantissa), normalised by its largest
 *       magnitude: {0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1, -0, -1/12, ..., -1}.
 *   levels_out: host, float[16], written.
 *   Errors: QK_ERR_INVALID_ARG for a null pointer or an unknown kind.
 */
qk_status qk_make_codebook(int32_t kind, float* levels_out);

/*
 * qk_quantize_blockwise — device.  [NF4] 【例子】, figure 2-2; [YOLO] sections
 * on 8-bit optimizers (a scale per block) and NF4.
 *   For each block j of the flattened input:
 *     absmax[j] = max |x_k| over the block (fp32, exact);
 *     t_k  = RN_fp32(x_k / absmax[j])   (IEEE division; t = +0 if absmax is 0);
 *     code = index of the level nearest to t_k, exactly; on a tie the smaller
 *            index wins;
 *   and the codes are packed two per byte, high nibble first.
 *   x:         device, [n] elements of x_dtype (QK_BF16, QK_F16 or QK_F32),
 *              16-byte aligned.
 *   n:         number of elements, 1..2^40.
 *   blocksize: 64, 128 or 256.
 *   levels:    host, float[16] in code order (any finite table in [-1, 1]
 *              whose distinct values have binary64-exact midpoints; both
 *              qk_make_codebook tables qualify).  Copied at the call.
 *   codes:     device, [ceil(n/2)] bytes, 4-byte aligned, written.
 *   absmax:    device, [ceil(n/blocksize)] fp32, 4-byte aligned, written.
 *   Errors: QK_ERR_INVALID_ARG (null / misaligned pointer, n < 1, bad block
 *   size or dtype, levels outside [-1, 1] or not finite); QK_ERR_UNSUPPORTED
 *   for a table whose lookup cannot be built exactly; QK_ERR_HIP on launch
 *   failure.
 */
qk_status qk_quantize_blockwise(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize,
                                const float* levels, uint8_t* codes, float* absmax, void* stream);

/*
 * qk_quantize_blockwise_grouped — device.  qk_quantize_blockwise of several
 * independent tensors (the weights of a layer) that share the input dtype, the
 * block size and the level table, same passages and the same definition per
 * tensor, in one launch for every run of up to 16 tensors of fewer than 2^26
 * elements (a larger tensor streams best in a launch of its own and gets one).
 * Each tensor's codes and absmax are bit-for-bit what qk_quantize_blockwise of
 * that tensor alone writes.
 *   tasks: host array of ntasks entries, each as the arguments of
 *     qk_quantize_blockwise: x (device, [n] elements, 16-byte aligned, read),
 *     n in 1..2^40, codes (device, [ceil(n/2)] bytes, 4-byte aligned, written),
 *     absmax (device, [ceil(n/blocksize)] fp32, 4-byte aligned, written).
 *   ntasks: 1..256.   x_dtype, blocksize, levels: as for qk_quantize_blockwise.
 *   No output may overlap another output or any input (else QK_ERR_INVALID_ARG).
 *   Errors: those of qk_quantize_blockwise.
 */
typedef struct qk_quant_task {
    const void* x;
    int64_t n;
    uint8_t* codes;
    float* absmax;
} qk_quant_task;

qk_status qk_quantize_blockwise_grouped(const qk_quant_task* tasks, int32_t ntasks, int32_t x_dtype,
                                        int32_t blocksize, const float* levels, void* stream);

/*
 * qk_double_quant_workspace_size — host.  Bytes of device workspace that
 * qk_double_quant needs for `nblocks` absmax values (a few bytes per 4096).
 */
qk_status qk_double_quant_workspace_size(int64_t nblocks, size_t* bytes);

/*
 * qk_double_quant — device.  [NF4] 【原理】② and 【代码】 (state2, offset);
 * [YOLO] section "Double quantization 連 scale 本身也壓縮".
 *     mean  = RN_fp32( T / nblocks ), T = the fp64 sum of absmax along a
 *             perfect binary tree (absmax zero-padded to the next power of two,
 *             neighbours added level by level), divided in fp64;
 *     c_j   = RN_fp32(absmax_j - mean);
 *     for each block d of dq_blocksize values (the last may be partial):
 *       s_d = max |c_j|,  scale[d] = RN_fp32(s_d / 127),
 *       q8_j = 0 if s_d == 0, else round-half-even( RN_fp32(RN_fp32(c_j / s_d) * 127) ).
 *   absmax:    device, [nblocks] fp32 (nblocks >= 1), 4-byte aligned.
 *   dq_blocksize: 256.
 *   q8:        device, [nblocks] int8, written.
 *   scale:     device, [ceil(nblocks/256)] fp32, written.
 *   mean:      device, [1] fp32, written.
 *   workspace: device, at least qk_double_quant_workspace_size() bytes,
 *              8-byte aligned; contents on entry are ignored.
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED (dq_blocksize != 256),
 *   QK_ERR_WORKSPACE, QK_ERR_HIP.
 */
qk_status qk_double_quant(const float* absmax, int64_t nblocks, int32_t dq_blocksize, int8_t* q8,
                          float* scale, float* mean, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * qk_double_quant_grouped — device.  qk_double_quant of several independent absmax
 * arrays (the weights of a layer quantized together), same passages and the same
 * definition per array, in two launches for every run of up to 16 arrays: one for
 * the fp64 tree partials of all of them, one for their int8 codes (an array of more
 * than 4096 * 4096 absmax values goes alone).  Each array's q8, scale and mean are
 * bit-for-bit what qk_double_quant of that array alone writes.
 *   tasks: host array of ntasks entries, each as the arguments of qk_double_quant:
 *     absmax: device, [nblocks] fp32 (nblocks >= 1), 4-byte aligned, read;
 *     q8: device, [nblocks] int8; scale: device, [ceil(nblocks/256)] fp32;
 *     mean: device, [1] fp32; all written, 4-byte aligned.
 *   ntasks: 1..256.   dq_blocksize: 256.
 *   workspace: device, at least qk_double_quant_grouped_workspace_size() bytes for
 *     the same tasks, 8-byte aligned; contents on entry are ignored.
 *   No output may overlap another output or any absmax (else QK_ERR_INVALID_ARG).
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED, QK_ERR_WORKSPACE, QK_ERR_HIP.
 */
typedef struct qk_dq_task {
    const float* absmax;
    int64_t nblocks;
    int8_t* q8;
    float* scale;
    float* mean;
} qk_dq_task;

/*
 * qk_double_quant_grouped_workspace_size — host.  Bytes of device workspace that
 * qk_double_quant_grouped needs for these tasks (only nblocks is read).
 */
qk_status qk_double_quant_grouped_workspace_size(const qk_dq_task* tasks, int32_t ntasks, size_t* bytes);

qk_status qk_double_quant_grouped(const qk_dq_task* tasks, int32_t ntasks, int32_t dq_blocksize, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * qk_state_init — host.  Fills a descriptor.  Pass absmax for a plain state,
 * or q8 / dq_scale / dq_mean (and absmax == NULL) for a nested one.
 *   levels: host float[16] in code order, copied.
 *   Errors: QK_ERR_INVALID_ARG (null state / codes / levels, rows or cols < 1,
 *   bad block size, neither or both absmax forms given).
 */
qk_status qk_state_init(qk_quant_state* st, int32_t codebook_kind, const float* levels,
                        int64_t rows, int64_t cols, int32_t blocksize, const uint8_t* codes,
                        const float* absmax, const int8_t* q8, const float* dq_scale,
                        const float* dq_mean);

/*
 * qk_dequantize — device.  [DEQ] section 5; [NF4] 【代码】.
 *     a'_j = absmax[j]                                   (plain), or
 *     a'_j = RN_fp32( RN_fp32(q8_j * dq_scale[d]) + dq_mean )   (nested);
 *     y_k  = RN_fp32( levels[code_k] * a'_{block(k)} )  (separate roundings, no FMA)
 *   written as fp32 or as bf16 (round to nearest even).  Signed zeros kept.
 *   st:  host pointer to a valid descriptor.
 *   out: device, [n] elements of out_dtype (QK_F32 or QK_BF16), 16-byte aligned.
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_HIP.
 */
qk_status qk_dequantize(const qk_quant_state* st, void* out, int32_t out_dtype, void* stream);

/*
 * qk_dequantize_grouped — device.  qk_dequantize of several states (the
 * weights of a layer) in as few launches as their level tables allow (up to 16
 * arrays of one table per launch; [DEQ] section 5).  Each out holds what
 * qk_dequantize of that state alone writes, bit for bit.
 *   tasks: host, ntasks (1..256) pairs of a valid descriptor and its output
 *     (device, [rows * cols] elements of out_dtype, 16-byte aligned, written);
 *     the outputs must be pairwise disjoint.
 *   out_dtype: QK_F32 or QK_BF16, for every task.
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_HIP (the argument
 *   checks run before anything is launched).
 */
typedef struct {
    const qk_quant_state* st;
    void* out;
} qk_dequant_task;

qk_status qk_dequantize_grouped(const qk_dequant_task* tasks, int32_t ntasks, int32_t out_dtype, void* stream);

/*
 * qk_gemv_nf4 — device.  Decode-time product with the dequantized weight:
 *     y[m, :] = x[m, :] · deq(W)^T,  m < M,
 *   [NF4] 【代码】 (4-bit linear forward: dequantize + matmul), [DEQ] section 5.
 *   The weight is dequantized inside the kernel and never written out.  The
 *   products use bf16 copies of the 16 levels, scaled by the block's absmax in
 *   fp32, with fp32 accumulation: the result agrees with the fp64 product on
 *   the bf16-dequantized weight to rel. Frobenius error <= 5e-3 and max error
 *   <= 2e-2 * max|ref|.
 *   x:  device, [M, K] bf16 row-major (K = st->cols), 16-byte aligned.
 *   M:  1..16.
 *   st: host pointer to a valid descriptor of W [N, K] (N = st->rows).
 *   y:  device, [M, N] bf16 row-major, written; 2-byte aligned.
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG (M outside 1..16, null or
 *   misaligned pointers), QK_ERR_HIP.
 */
qk_status qk_gemv_nf4(const void* x, int32_t M, const qk_quant_state* st, void* y, void* stream);

/*
 * qk_gemv_nf4_grouped — device.  qk_gemv_nf4 of several weights, each with its own
 * x and y and the same M, in as few launches as possible: one per run of up to 16
 * weights that share the level table, block size and nesting (a decode step's
 * q / k / v, or gate / up, or a whole layer when their inputs are ready together).
 * Each y is bit-for-bit what qk_gemv_nf4 of that weight alone writes.
 *   tasks: host array of ntasks entries
 *     x:  device, [M, K] bf16 row-major (K = st->cols), 16-byte aligned;
 *     st: host pointer to a valid descriptor of W [N, K];
 *     y:  device, [M, N] bf16 row-major, written; 2-byte aligned.
 *   ntasks: 1..256.   M: 1..16.
 *   No y may overlap another task's y or any task's x (else QK_ERR_INVALID_ARG).
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_HIP.
 */
typedef struct qk_gemv_task {
    const void* x;
    const qk_quant_state* st;
    void* y;
} qk_gemv_task;

qk_status qk_gemv_nf4_grouped(const qk_gemv_task* tasks, int32_t ntasks, int32_t M, void* stream);

/*
 * qk_gemm_nf4_workspace_size — host.  Bytes of device workspace qk_gemm_nf4
 * needs for M token rows and LoRA rank r (0 when r == 0: no workspace).
 */
qk_status qk_gemm_nf4_workspace_size(int64_t M, int32_t r, size_t* bytes);

/*
 * qk_gemm_nf4 — device.  Prefill / training forward of a frozen 4-bit base
 * layer with an unmerged LoRA adapter ([DEQ] sections 2-2 and 8; [NF4] §2.2):
 *     Y = X · deq(W)^T + lora_scale · (X · A) · B
 *   The weight is dequantized tile by tile to bf16 exactly as qk_dequantize
 *   would write it and multiplied on bf16 matrix cores with fp32 accumulation.
 *   The rank-r LoRA term: lora_scale · X · A is formed once per call (fp32, in
 *   the workspace), and its product with B is added to the accumulators in the
 *   GEMM epilogue.  Agreement with the fp64 reference: rel. Frobenius <= 5e-3,
 *   max error <= 2e-2 * max|ref|.
 *   X: device, [M, K] bf16 row-major, K = st->cols.
 *   M: >= 1.
 *   A: device, [K, r] bf16 row-major, or NULL (no LoRA term).
 *   B: device, [r, N] bf16 row-major, or NULL (no LoRA term).
 *   r: LoRA rank, 1..64 when A and B are given (ignored otherwise).
 *   lora_scale: alpha / r.
 *   Y: device, [M, N] bf16 row-major, written.
 *   workspace: device, >= qk_gemm_nf4_workspace_size(M, r) bytes, 16-byte
 *     aligned (may be NULL when A and B are NULL); contents on entry ignored.
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_WORKSPACE, QK_ERR_HIP.
 */
qk_status qk_gemm_nf4(const void* X, int64_t M, const qk_quant_state* st, const void* A,
                      const void* B, int32_t r, float lora_scale, void* Y, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * qk_gemm_nf4_grouped — device.  Several qk_gemm_nf4 products (the weights of
 * a layer, each with its own X, adapter and Y) in as few launches as their
 * shapes allow ([DEQ] sections 2-2 and 8; [NF4] §2.2).  Each Y is the one
 * qk_gemm_nf4 of that task alone writes, bit for bit.  The tasks whose weights
 * the 256 x 256 kernel takes (K a multiple of 64 and of the block size, 16-byte
 * aligned X and codes) and that share the rank class ceil(r / 16) and the
 * nesting run in one launch (up to 8 per launch), longest rows first, after
 * their LoRA pre-passes; the others run one by one.  One launch packs the tiles
 * of all its GEMMs, so no GEMM's partial last round leaves CUs idle.
 *   tasks: host, ntasks (1..256) descriptors; X, M, st, A, B, r, lora_scale
 *     and Y as for qk_gemm_nf4.  Every Y must be disjoint from the other Ys,
 *     from every X and from the workspace.
 *   workspace: device, >= qk_gemm_nf4_grouped_workspace_size bytes, 16-byte
 *     aligned (may be NULL when no task has an adapter); contents ignored.
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_WORKSPACE, QK_ERR_HIP
 *   (the argument checks run before anything is launched).
 */
typedef struct {
    const void* X;               /* device, [M, K] bf16 */
    int64_t M;
    const qk_quant_state* st;    /* the weight, [N, K] */
    const void* A;               /* device, [K, r] bf16, or NULL */
    const void* B;               /* device, [r, N] bf16, or NULL */
    int32_t r;
    float lora_scale;
    void* Y;                     /* device, [M, N] bf16, written */
} qk_gemm_task;

/* Bytes of workspace qk_gemm_nf4_grouped needs for these tasks (the sum of the
 * tasks' LoRA partials, each rounded up to 256 bytes).  Host only. */
qk_status qk_gemm_nf4_grouped_workspace_size(const qk_gemm_task* tasks, int32_t ntasks, size_t* bytes);

qk_status qk_gemm_nf4_grouped(const qk_gemm_task* tasks, int32_t ntasks, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * qk_gemm_nf4_noalloc — device.  qk_gemm_nf4 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and the same result, bit for bit, as
 * qk_gemm_nf4 with a workspace, but the LoRA partials live in a static device
 * array of the library (8 MiB per device, held until the process ends), so the
 * call takes no workspace and allocates nothing.
 *   X, M, st, A, B, r, lora_scale, Y: as for qk_gemm_nf4.
 *   Limit: with an adapter, M * 16 * ceil(r / 16) <= 262144 (for instance
 *   M <= 16384 at r <= 16, M <= 4096 at r <= 64); larger calls are refused
 *   with QK_ERR_WORKSPACE and launch nothing.
 *   Every call on one device shares its array: calls that overlap on one device
 *   (on different streams, or from different threads) race and give undefined
 *   results; calls in one stream order are safe.  The first call on a device
 *   looks up the array's address (hipGetSymbolAddress), so make it once before
 *   graph capture.
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_WORKSPACE, QK_ERR_HIP.
 */
qk_status qk_gemm_nf4_noalloc(const void* X, int64_t M, const qk_quant_state* st, const void* A,
                              const void* B, int32_t r, float lora_scale, void* Y, void* stream);

/*
 * qk_lora_merge — device.  Merges a LoRA adapter into the dequantized weight,
 * [DEQ] section 8 (merge: dequantize the 4-bit weight to BF16, add the LoRA
 * product, W_new is BF16; requantize it with qk_quantize_blockwise when a
 * 4-bit weight is wanted) and section 9 (the QLoRA life cycle):
 *     D[n, k] = bf16( RN_fp32(levels[code] * a') )      (qk_dequantize's bf16 value)
 *     P[n, k] = sum_{j = 0 .. r-1} B[j, n] * A[k, j]    (fp32, j increasing; the
 *                                                        products of bf16 values are exact)
 *     out[n, k] = bf16( RN_fp32( D + RN_fp32(lora_scale * P) ) )   (round to nearest even)
 *   Bit-exact: the same inputs give the same bits on every call.
 *   st: host pointer to a valid descriptor of W [N, K].
 *   A:  device, [K, r] bf16 row-major.   B: device, [r, N] bf16 row-major.
 *   r:  1..1024.   lora_scale: finite (alpha / r).
 *   out: device, [N, K] bf16 row-major, written (2-byte aligned; 16-byte alignment
 *     and K % 8 == 0 select the vectorized path).
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_HIP.
 */
qk_status qk_lora_merge(const qk_quant_state* st, const void* A, const void* B, int32_t r,
                        float lora_scale, void* out, void* stream);

/*
 * qk_qlora_backward_workspace_size — host.  Bytes of device workspace
 * qk_qlora_backward needs for M token rows, the weight of `st` and LoRA rank r
 * (0 when r == 0).
 */
qk_status qk_qlora_backward_workspace_size(int64_t M, const qk_quant_state* st, int32_t r,
                                           size_t* bytes);

/*
 * qk_qlora_backward — device.  Backward of the layer qk_gemm_nf4 computes,
 * Y = X · deq(W)^T + s · (X · A) · B, for an upstream gradient dY; the 4-bit
 * base stays frozen and is dequantized tile by tile as in the forward ([YOLO]
 * section "QLoRA 把 frozen 4-bit base 與可訓練 adapter 分開": dequantized in the
 * forward and the backward pass; [DEQ] section 4: the INT4 base is frozen, only
 * the BF16 A and B train; section 5: the base is restored to BF16 per layer):
 *     G  = dY · B^T
 *     dX = dY · deq(W) + s · G · A^T        (bf16)
 *     dA = s · X^T · G                      (fp32)
 *     dB = s · (X · A)^T · dY               (fp32)
 *   Agreement with the fp64 reference: rel. Frobenius <= 5e-3 and max error
 *   <= 2e-2 * max|ref| for each output.  Deterministic.
 *   dY: device, [M, N] bf16 row-major (N = st->rows), 16-byte aligned.
 *   X:  device, [M, K] bf16 row-major (K = st->cols), 16-byte aligned; needed
 *       only with an adapter.
 *   A, B: device, [K, r] and [r, N] bf16 row-major, or both NULL (dX only).
 *   r: 1..64 with an adapter.   lora_scale: finite (alpha / r).
 *   dX: device, [M, K] bf16, written.   dA: device, [K, r] fp32, written.
 *   dB: device, [r, N] fp32, written (dA, dB ignored without an adapter).
 *   workspace: device, >= qk_qlora_backward_workspace_size(M, st, r) bytes,
 *     16-byte aligned (NULL allowed without an adapter).
 *   N and K must be multiples of 64 (else QK_ERR_UNSUPPORTED).
 *   Errors: QK_ERR_BAD_STATE, QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED,
 *   QK_ERR_WORKSPACE, QK_ERR_HIP.
 */
qk_status qk_qlora_backward(const void* dY, int64_t M, const qk_quant_state* st, const void* X,
                            const void* A, const void* B, int32_t r, float lora_scale, void* dX,
                            float* dA, float* dB, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * qk_make_dynamic_map — host.  [OPT8]: the page names the map and its
 * properties but gives no construction; the levels are equal-mass quantiles,
 *   signed   (is_signed != 0): levels[i] = RN_fp32( Phi^-1((2i+1)/512) / Phi^-1(511/512) )
 *   unsigned (is_signed == 0): levels[i] = RN_fp32( Phi^-1(1/2 + (2i+1)/1024) / Phi^-1(1/2 + 511/1024) )
 *   i = 0..255, increasing; the signed map is antisymmetric with levels[0] = -1,
 *   levels[255] = 1 and no zero level; the unsigned map lies in (0, 1].
 *   levels_out: host, float[256], written.
 *   Errors: QK_ERR_INVALID_ARG (NULL levels_out).
 */
qk_status qk_make_dynamic_map(int32_t is_signed, float* levels_out);

/*
 * qk_quantize_blockwise_8bit — device.  [OPT8]: per block j of `blocksize`
 * consecutive elements of the flattened x (the last block may be partial),
 *   absmax[j] = max |x_k|  (fp32),
 *   t_k = RN_fp32(x_k / absmax[j])  (IEEE division; t = +0 when absmax[j] == 0),
 *   codes[k] = the index of the nearest level to t_k, ties to the smaller index.
 *   x:         device, [n] elements of x_dtype (QK_BF16, QK_F16 or QK_F32), 16-byte aligned.
 *   n:         >= 1.   blocksize: 256, 512, 1024, 2048 or 4096 (2048 in [OPT8]).
 *   levels:    host, float[256] in [-1, 1], code order (any order; ties between
 *              equal values go to the smaller code); copied at the call.
 *              Thresholds closer than 1/1024 are refused (QK_ERR_UNSUPPORTED);
 *              both qk_make_dynamic_map tables qualify.
 *   codes:     device, uint8[n], one code per byte, 8-byte aligned, written.
 *   absmax:    device, float[ceil(n / blocksize)], 4-byte aligned, written.
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED, QK_ERR_NO_DEVICE, QK_ERR_HIP.
 */
qk_status qk_quantize_blockwise_8bit(const void* x, int32_t x_dtype, int64_t n, int32_t blocksize,
                                     const float* levels, uint8_t* codes, float* absmax, void* stream);

/*
 * qk_dequantize_blockwise_8bit — device.  [OPT8]: out[k] = RN_fp32(levels[codes[k]] *
 *   absmax[k / blocksize]), written as fp32 or as bf16 (RNE).
 *   codes:  device, uint8[n], 8-byte aligned.   absmax: device, float[ceil(n / blocksize)].
 *   n >= 1; blocksize as for quantize; levels: host, float[256], copied at the call.
 *   out:    device, [n] elements of out_dtype (QK_F32 or QK_BF16), 16-byte aligned, written.
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_NO_DEVICE, QK_ERR_HIP.
 */
qk_status qk_dequantize_blockwise_8bit(const uint8_t* codes, const float* absmax, int64_t n, int32_t blocksize,
                                       const float* levels, void* out, int32_t out_dtype, void* stream);

/*
 * qk_int8_quantize_rows — device.  [INT8] vector-wise quantization: for each row r
 * of the row-major matrix x [rows, cols],
 *   absmax[r] = max |x[r, k]| over the columns k with skip_cols[k] == 0,
 *   q[r, k]   = rint_even( RN_fp32( RN_fp32(x[r, k] / absmax[r]) * 127 ) ) in [-127, 127],
 *               0 when absmax[r] == 0 or skip_cols[k] != 0.
 *   Used for the weight (CB = q, SCB = absmax, skip_cols NULL) and for the
 *   activations (skip_cols = the outlier flags of qk_int8_outlier_columns).
 *   x: device, x_dtype QK_F16, QK_BF16 or QK_F32, 16-byte aligned.   rows, cols >= 1, cols % 8 == 0.
 *   skip_cols: device, uint8[cols], 8-byte aligned, or NULL.
 *   q: device, int8[rows * cols], 8-byte aligned, written.   absmax: device, float[rows], written.
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_NO_DEVICE, QK_ERR_HIP.
 */
qk_status qk_int8_quantize_rows(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, const uint8_t* skip_cols,
                                int8_t* q, float* absmax, void* stream);

/*
 * qk_int8_outlier_columns — device.  [INT8] 【例子】 and figure 2-1: column k of x
 * [M, K] is an outlier when max_m |x[m, k]| > threshold (strictly; none when
 * threshold == 0).
 *   x: device, x_dtype as above, 16-byte aligned; M >= 1, K >= 1, K % 8 == 0.
 *   threshold: finite, >= 0.
 *   colmax: device, float[K], written (the column maxima).
 *   flags:  device, uint8[K], written (1 = outlier).
 *   idx:    device, int32[K]; its first *count entries are written with the
 *           outlier columns in increasing order.
 *   count:  device, int32[1], written.  Deterministic.
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_NO_DEVICE, QK_ERR_HIP.
 */
qk_status qk_int8_outlier_columns(const void* x, int32_t x_dtype, int64_t M, int64_t K, float threshold, float* colmax,
                                  uint8_t* flags, int32_t* idx, int32_t* count, void* stream);

/*
 * qk_int8_matmul — device.  [INT8] mixed-precision decomposition, for X [M, K]
 * (fp16) against the int8 weight (CB [N, K], SCB [N]):
 *   Y[m, n] = sum_{k not outlier} Xq[m, k] CB[n, k] * SX[m] * SCB[n] / 127^2
 *           + sum_{k outlier} X[m, k] * fp16(CB[n, k] * SCB[n] / 127),
 *   the int8 products summed exactly in int32, the rest in fp32; Y is written
 *   in fp16.  Agreement with the fp64 reference: rel. Frobenius <= 5e-3, max
 *   error <= 2e-2 * max |ref|.
 *   Xq, SX: device, from qk_int8_quantize_rows of X with the outlier columns
 *           skipped (int8 [M, K] 16-byte aligned; float[M]).
 *   CB, SCB: device, from qk_int8_quantize_rows of W [N, K] (int8 [N, K] 16-byte aligned; float[N]).
 *   M, N >= 1; K >= 16, K % 16 == 0.
 *   X, outlier_idx, outlier_count: device, the fp16 X [M, K], and idx / count from
 *           qk_int8_outlier_columns; all three NULL for no outlier path.
 *   Y: device, fp16 [M, N], written.
 *   Errors: QK_ERR_INVALID_ARG, QK_ERR_NO_DEVICE, QK_ERR_HIP.
 */
qk_status qk_int8_matmul(const int8_t* Xq, const float* SX, const int8_t* CB, const float* SCB, int64_t M, int64_t N,
                         int64_t K, const void* X, const int32_t* outlier_idx, const int32_t* outlier_count, void* Y,
                         void* stream);

/* Message for the calling thread's last failed call ("" if none).  The
 * string stays valid until the thread's next qk_* call. */
const char* qk_last_error(void);

/* Library version string, e.g. "qk 0.1.0 gfx950". */
const char* qk_version(void);

/* Which kernel variant each call uses, for logs and benchmarks. */
const char* qk_backend_info(void);

#ifdef __cplusplus
}
#endif

#endif /* QK_H */
