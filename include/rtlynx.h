/*
 * rtlynx.h - C ABI of librtlynx, an online 2:4 activation-sparse linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (RT-Lynx, arXiv 2605.26632):
 *
 *   Y = S(X) W^T + alpha * ((X - S(X)) A^T) B^T
 *
 * S(X) is computed online, per token (row of X):
 *   - in every group of 4 consecutive input channels the two entries of
 *     largest magnitude are kept and the other two are pruned
 *     (ai-feeds summary, section 方法 / 输入与稀疏化策略: a 2:4 pattern on the
 *     activations; qingkeai article, section 01: 2 non-zeros in every 4
 *     consecutive elements; section 03.1: Top-K selection).  Equal magnitudes
 *     are resolved toward the lower channel index, so the kept set is unique;
 *   - the kept entries are multiplied by s = (L1 of the row) / (L1 of the
 *     kept entries), which hands the pruned L1 mass back to the kept values in
 *     proportion to their magnitude (ai-feeds summary, 方法 / 核心模块 1,
 *     norm-compensated sparsification; qingkeai article, section 03.1).
 *     s = 1 for an all-zero row;
 *   - W is the dense frozen weight (qingkeai article, section 02:
 *     Y = S(X) W^T); the rank-r LoRA branch (A, B) acts on the pruned
 *     residual X - S(X) (qingkeai article, section 03.2; rank 64 in the
 *     neuraltrendhub summary, "What the paper found").
 *
 * Common conventions for every entry point:
 *   - bf16 tensors are passed as raw 16-bit words (uint16_t), row-major,
 *     densely packed (row stride = number of columns).
 *   - Every tensor pointer is device memory owned by the caller.  The library
 *     allocates nothing and keeps no pointer after a call returns.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise.  Outputs must not alias inputs.
 *   - The kernels run on the current device (hipSetDevice), and hip_stream
 *     must belong to it, else RTL_ERR_STREAM_DEVICE; every tensor pointer
 *     must be memory of that device.
 *   - Host threads may call the library concurrently: its only state is a
 *     per-device record of the architecture check, written atomically.  Calls
 *     that can run at the same time on the GPU (different streams with no
 *     ordering between them) must not share a workspace or an output buffer.
 *   - Every base pointer must be 16-byte aligned.
 *   - The linear-layer entry points address every tensor and every workspace
 *     region with 32-bit offsets: each of X, W, Y, A, B and the workspace
 *     regions must be smaller than 2 GiB (2^31 bytes), else
 *     RTL_ERR_BAD_SHAPE.  Larger token counts are processed in row chunks.
 *   - Arguments are validated before any HIP call; on error nothing is
 *     launched and nothing is written.  The library keeps no sticky error
 *     state: a failed call leaves it usable.
 *   - Only gfx950 devices are supported: any other device gives
 *     RTL_ERR_UNSUPPORTED_ARCH, no device gives RTL_ERR_NO_DEVICE.
 *   - No C++ exception crosses this interface.
 */
#ifndef RTLYNX_H
#define RTLYNX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RTL_OK = 0,
  RTL_ERR_NULL_POINTER = 1,      /* a required pointer is NULL              */
  RTL_ERR_BAD_SHAPE = 2,         /* negative size, K % 4 != 0, K == 0, 2 GiB */
  RTL_ERR_MISALIGNED = 3,        /* a base pointer is not 16-byte aligned    */
  RTL_ERR_WORKSPACE = 4,         /* workspace missing or too small           */
  RTL_ERR_NO_DEVICE = 5,         /* no HIP device is visible                 */
  RTL_ERR_UNSUPPORTED_ARCH = 6,  /* the current device is not gfx950         */
  RTL_ERR_HIP = 7,               /* a HIP runtime call or launch failed      */
  RTL_ERR_BAD_FLAGS = 8,         /* unknown bits in a flags argument         */
  RTL_ERR_STREAM_DEVICE = 9      /* hip_stream is not on the current device  */
} rtl_status;

/* rtl_sparsify_2of4 flag: store vals = bf16_rne(s * x) (the compensated
 * values) instead of exact copies of x. */
#define RTL_FOLD_SCALE 0x1u

/* Largest LoRA rank the fused path accepts. */
#define RTL_MAX_LORA_RANK 128

/*
 * rtl_sparsify_2of4 - mask, compensation scale and compression of X.
 *
 * The 2:4 pattern decision, Top-K selection and activation compression of the
 * fused path (qingkeai article, section 04), written out to HBM in the
 * library's canonical compressed format:
 *
 *   x      [M, K]            bf16, input activations, K % 4 == 0, K >= 4.
 *   vals   [M, K/2]          bf16, output: group g's two kept words at
 *                            columns 2g and 2g+1, lower channel first; exact
 *                            copies of x unless flags has RTL_FOLD_SCALE.
 *   idx    [M, ceil(K/8)]    uint8, output: group g's code
 *                            idx0 | idx1 << 2 (idx0 < idx1 the kept in-group
 *                            positions) in byte g/2, low nibble for even g,
 *                            high nibble for odd g; when K/4 is odd the last
 *                            byte's high nibble is 0.
 *   scale  [M]               fp32, output, may be NULL: the per-token s.
 *   flags                    0 or RTL_FOLD_SCALE.
 *
 * M == 0 is a no-op.  The base pointers x, vals, idx and scale (when not
 * NULL) must be 16-byte aligned; rows of vals and idx need not be.
 */
rtl_status rtl_sparsify_2of4(const uint16_t* x, int64_t M, int64_t K,
                             uint16_t* vals, uint8_t* idx, float* scale,
                             uint32_t flags, void* hip_stream);

/*
 * rtl_sparse_linear_workspace_bytes - device workspace rtl_sparse_linear needs
 * for M tokens, K input channels and LoRA rank r (the compressed activation in
 * the matrix-core operand order, the per-token scale and the LoRA-down
 * product).  Returns 0 for invalid sizes.
 */
size_t rtl_sparse_linear_workspace_bytes(int64_t M, int64_t K, int64_t r);

/*
 * rtl_sparse_linear - the fused online 2:4 activation-sparse linear layer:
 * pattern decision, Top-K, compression, sparse GEMM on the structured-sparse
 * matrix cores, and the LoRA residual branch (qingkeai article, sections 02,
 * 03 and 04).
 *
 *   x         [M, K]   bf16 activations (tokens x input channels).
 *   w         [N, K]   bf16 dense frozen weight (nn.Linear layout).
 *   lora_a    [r, K]   bf16 LoRA down factor; required when r > 0,
 *                      ignored when r == 0.
 *   lora_b    [N, r]   bf16 LoRA up factor; same rule as lora_a.
 *   lora_scale         alpha, multiplies the LoRA branch.
 *   y         [M, N]   bf16 output, fp32 accumulation rounded to nearest even.
 *   workspace          device scratch of at least
 *                      rtl_sparse_linear_workspace_bytes(M, K, r) bytes,
 *                      16-byte aligned.  Its contents are overwritten.
 *
 * K % 4 == 0, K >= 4, 0 <= r <= RTL_MAX_LORA_RANK.  M == 0 or N == 0 is a
 * no-op.  M, N and K need not be tile multiples.
 */
rtl_status rtl_sparse_linear(const uint16_t* x, const uint16_t* w,
                             const uint16_t* lora_a, const uint16_t* lora_b,
                             int64_t M, int64_t N, int64_t K, int64_t r,
                             float lora_scale, uint16_t* y,
                             void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/* Size of the device scratch array that rtl_sparse_linear_noalloc uses in
 * place of a caller workspace (64 MiB; one copy per GPU the library runs
 * on, held until the process ends). */
#define RTL_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * rtl_sparse_linear_noalloc - rtl_sparse_linear for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as rtl_sparse_linear without the workspace: the
 * workspace is a fixed device array inside the library, one per GPU,
 * RTL_NOALLOC_SCRATCH_BYTES long.  A layer whose
 * rtl_sparse_linear_workspace_bytes(M, K, r) exceeds that gives
 * RTL_ERR_WORKSPACE (e.g. M = 9216, K = 3072, r = 64 needs 34 MB; M = 4096,
 * K = 12288, r = 64 needs 58 MB).  The call allocates nothing, through HIP or
 * otherwise.  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents: calls that can overlap on one GPU (different streams
 * without ordering between them, or several host threads) race on it and
 * must be serialised by the caller.
 */
rtl_status rtl_sparse_linear_noalloc(const uint16_t* x, const uint16_t* w,
                                     const uint16_t* lora_a, const uint16_t* lora_b,
                                     int64_t M, int64_t N, int64_t K, int64_t r,
                                     float lora_scale, uint16_t* y, void* hip_stream);

/*
 * rtl_sparse_linear_prepare / rtl_sparse_linear_apply - the two halves of
 * rtl_sparse_linear, for callers that feed one activation to several weights
 * (e.g. projections that share an input) or that time the halves apart.
 *
 * prepare reads x once: the 2:4 pattern decision, Top-K, norm-compensation
 * scale, compression into the structured-sparse matrix-core operand order
 * ("activation compression" and "layout generation", qingkeai article,
 * section 04) and the LoRA-down product of the pruned residual (section
 * 03.2), all written into `workspace`.  apply runs the sparse GEMM against w
 * and the scale + LoRA-up epilogue, reading only the workspace, w and lora_b.
 *
 * Arguments mean what they mean for rtl_sparse_linear.  apply must see the
 * same M, K and r as the prepare that filled the workspace, and the
 * workspace must not be modified in between; apply may be called any number
 * of times with different w / lora_b / N.  lora_scale is applied in prepare.
 */
rtl_status rtl_sparse_linear_prepare(const uint16_t* x, const uint16_t* lora_a,
                                     int64_t M, int64_t K, int64_t r, float lora_scale,
                                     void* workspace, size_t workspace_bytes,
                                     void* hip_stream);

rtl_status rtl_sparse_linear_apply(const void* workspace, size_t workspace_bytes,
                                   const uint16_t* w, const uint16_t* lora_b,
                                   int64_t M, int64_t N, int64_t K, int64_t r,
                                   uint16_t* y, void* hip_stream);

/*
 * Variants of the layer the pages leave open (for rtl_sparse_linear_prepare_variant).
 * Compensation -- how the pruned L1 mass returns to the kept values (ai-feeds
 * summary, 核心模块 1, and qingkeai article, section 03.1, give the idea, not
 * the granularity):
 *   RTL_COMP_TOKEN   per token, s = (Lk + Lp) / Lk, applied to the fp32
 *                    accumulators (the default; what rtl_sparse_linear does);
 *   RTL_COMP_NONE    no compensation, s = 1;
 *   RTL_COMP_TENSOR  one factor for the whole activation,
 *                    (sum over tokens of Lk + Lp) / (sum of Lk), 1 if that is 0;
 *   RTL_COMP_GROUP   per group of 4, (L1 of the group) / (L1 of its kept pair),
 *                    multiplied into the kept values, which are then rounded to
 *                    bf16 (a factor that varies along K can only live in the
 *                    compressed operand); s = 1.
 * LoRA input R of T = R A^T (qingkeai article, section 03.2: the branch
 * restores the pruned information):
 *   RTL_LORA_RESIDUAL  R = X - S(X) (the default);
 *   RTL_LORA_PRUNED    R = (1 - M) * X, the pruned values;
 *   RTL_LORA_INPUT     R = X.
 * variant = one RTL_COMP_* | one RTL_LORA_*.
 */
#define RTL_COMP_TOKEN 0x0u
#define RTL_COMP_NONE 0x1u
#define RTL_COMP_TENSOR 0x2u
#define RTL_COMP_GROUP 0x3u
#define RTL_LORA_RESIDUAL 0x0u
#define RTL_LORA_PRUNED 0x4u
#define RTL_LORA_INPUT 0x8u

/*
 * rtl_sparse_linear_prepare_variant - rtl_sparse_linear_prepare for one of
 * the variants above; rtl_sparse_linear_apply then completes the layer
 *
 *   y = bf16( S(X) W^T + lora_scale * (R A^T) B^T )
 *
 * with S and R as the variant defines them.  Arguments, workspace size and
 * errors as for rtl_sparse_linear_prepare; an unknown bit in variant, or
 * both RTL_LORA_* bits, gives RTL_ERR_BAD_FLAGS.  RTL_COMP_TENSOR runs two
 * more kernels on the stream first (the activation's L1 statistics, read from
 * x, and their fixed-order fp64 sum), so the result is deterministic.
 */
rtl_status rtl_sparse_linear_prepare_variant(const uint16_t* x, const uint16_t* lora_a,
                                             int64_t M, int64_t K, int64_t r, float lora_scale,
                                             uint32_t variant, void* workspace,
                                             size_t workspace_bytes, void* hip_stream);

/*
 * rtl_sparse_linear_compressed - the structured-sparse GEMM on an activation
 * already compressed in the canonical format of rtl_sparsify_2of4 (compress
 * once, multiply by any number of weights; also the unfused form of the layer,
 * sparsify then GEMM, that the qingkeai article, section 04, contrasts with
 * the fused kernel):
 *
 *   y = bf16( scale[m] * sum_k decompress(vals, idx)[m, k] * w[n, k] )
 *
 *   vals   [M, K/2] bf16, idx [M, ceil(K/8)] bytes: exactly as rtl_sparsify_2of4
 *          writes them (idx nibble idx0 | idx1 << 2, idx0 < idx1, even group
 *          in the low nibble; the values multiply W at channels 4g + idx0 and
 *          4g + idx1 of group g).
 *   scale  [M] fp32 per-token factor applied to the fp32 accumulators, or NULL
 *          for 1 (e.g. values stored with RTL_FOLD_SCALE).
 *   w      [N, K] bf16, y [M, N] bf16 (outputs; caller-owned device memory).
 *   workspace  device memory of rtl_sparse_linear_workspace_bytes(M, K, 0)
 *          bytes, overwritten (the operand reordered for the matrix cores).
 *
 * There is no LoRA branch (the canonical format carries no LoRA-down).  Same
 * shape, alignment, ownership, stream and error rules as rtl_sparse_linear
 * (r = 0); a code of 0 in idx is accepted (both positions 0) and contributes
 * whatever its two values give.
 */
rtl_status rtl_sparse_linear_compressed(const uint16_t* vals, const uint8_t* idx,
                                        const float* scale, const uint16_t* w,
                                        int64_t M, int64_t N, int64_t K, uint16_t* y,
                                        void* workspace, size_t workspace_bytes,
                                        void* hip_stream);

/*
 * rtl_dense_linear - the dense baseline Y = X W^T (the denominator of the
 * speedups the pages quote, qingkeai article, section 05), bf16 inputs, fp32
 * accumulation on the dense matrix cores, bf16 output rounded to nearest even.
 *
 *   x [M, K], w [N, K], y [M, N].  K % 4 == 0, K >= 4.  M == 0 or N == 0 is
 *   a no-op.
 */
rtl_status rtl_dense_linear(const uint16_t* x, const uint16_t* w,
                            int64_t M, int64_t N, int64_t K,
                            uint16_t* y, void* hip_stream);

/* Static, NUL-terminated description of a status code. */
const char* rtl_status_string(rtl_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int rtl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RTLYNX_H */
