/*
 * rtlynx_layers.h - per-layer dispatch of librtlynx: selective layer
 * skipping.
 *
 * Not every linear layer of a diffusion transformer is equally robust to the
 * online 2:4 sparsification: the RT-Lynx pages skip it on some sensitive
 * layers of single-stream models such as FLUX.1-dev and Z-Image, or give
 * different layers different sparsification strategies (ai-feeds summary,
 * 方法 / 核心模块 3, selective layer skipping; qingkeai article, section 03,
 * item 3).  Which layers those are depends on the model and its weights; the
 * caller states it in a table of per-layer modes, and rtl_layer_linear runs
 * each call the way its layer's mode says.
 *
 * A skipped layer computes the dense product Y = X W^T: without
 * sparsification S(X) = X, so the LoRA branch, which acts on the pruned
 * residual X - S(X), contributes nothing.  The call is then exactly
 * rtl_dense_linear.
 */
#ifndef RTLYNX_LAYERS_H
#define RTLYNX_LAYERS_H

#include "rtlynx.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Per-layer mode: RTL_LAYER_DENSE skips the sparsification (dense product),
 * any other value is a sparsification variant of
 * rtl_sparse_linear_prepare_variant (one RTL_COMP_* | one RTL_LORA_*;
 * 0 = the default layer of rtl_sparse_linear). */
#define RTL_LAYER_DENSE 0x100u

/* Hint OR-ed into a mode: the layer's weights are not expected in the
 * caches (a model whose layers each run once per forward pass streams its
 * weights through the 256 MB last-level cache between two calls of the same
 * layer).  A sparse layer then runs the GEMM instance that probes the W
 * lines into L2 a few k-steps ahead of their copies: the same arithmetic and
 * the same output bits, faster with W in HBM only, slower with W already
 * cached.  Applies to the ring shapes (r % 8 == 0, K % 8 == 0); dense
 * layers and other shapes ignore it. */
#define RTL_LAYER_STREAM_W 0x200u

/*
 * rtl_layer_linear - one linear layer of a model under a layer-skip policy.
 *
 *   layer_modes  host array of num_layers modes (RTL_LAYER_DENSE or a
 *                variant), owned by the caller, read during the call only.
 *   layer        index of this layer, 0 <= layer < num_layers.
 *   the rest     as for rtl_sparse_linear.  For a dense layer lora_a,
 *                lora_b, lora_scale and the workspace are ignored (may be
 *                NULL / 0) and the call is rtl_dense_linear(x, w, M, N, K,
 *                y, hip_stream); for a sparse layer it is rtl_sparse_linear
 *                (variant 0) or rtl_sparse_linear_prepare_variant followed by
 *                rtl_sparse_linear_apply, with their arguments, rules and
 *                errors.
 *
 * Errors: layer_modes NULL with num_layers > 0 gives RTL_ERR_NULL_POINTER;
 * num_layers < 0 or layer outside [0, num_layers) gives RTL_ERR_BAD_SHAPE; a
 * mode that is neither RTL_LAYER_DENSE nor a valid variant, with or without
 * RTL_LAYER_STREAM_W, gives RTL_ERR_BAD_FLAGS.  All before any HIP call.
 */
rtl_status rtl_layer_linear(const uint32_t* layer_modes, int64_t num_layers, int64_t layer,
                            const uint16_t* x, const uint16_t* w,
                            const uint16_t* lora_a, const uint16_t* lora_b,
                            int64_t M, int64_t N, int64_t K, int64_t r,
                            float lora_scale, uint16_t* y,
                            void* workspace, size_t workspace_bytes,
                            void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RTLYNX_LAYERS_H */
