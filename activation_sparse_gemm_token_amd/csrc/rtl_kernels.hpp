// Launch wrappers of librtlynx's kernels (internal; the public interface is
// include/rtlynx.h).  Each returns the status of its own launches (the
// first that failed), never the thread's earlier error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtl {

// compute_units: the device's CU count (one or two wavefronts per row).
hipError_t launch_sparsify_2of4(const uint16_t* x, int64_t M, int64_t K, uint16_t* vals,
                                uint8_t* idx, float* scale, bool fold, int compute_units,
                                hipStream_t stream);

// Pre-pass of the fused path: selection, compression into the structured-
// sparse matrix-core operand order, per-token scale, LoRA-down product.
hipError_t launch_prepass(const uint16_t* x, const uint16_t* lora_a, int64_t M, int64_t K,
                          int64_t r, float lora_scale, void* workspace, hipStream_t stream,
                          int comp = 0, int lora = 0);

// Sparse GEMM on the compressed operand plus the scale and LoRA-up epilogue.
// `compute_units`: the device's CU count (the persistent grid's size).
// tile_n: 256 or 192 output columns per tile, 0 to let
// sparse_gemm_tile_n choose (the one that fills the CUs at lower cost).
// prefetch_w: probe W lines into L2 a few steps ahead of their copies (for
// weights not expected in the caches; the ring shapes, r % 8 == 0 and
// K % 8 == 0, only).
hipError_t launch_sparse_gemm(const void* workspace, const uint16_t* w, const uint16_t* lora_b,
                              int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y,
                              int compute_units, hipStream_t stream, int tile_n = 0,
                              bool prefetch_w = false);
int sparse_gemm_tile_n(int64_t M, int64_t N, int64_t K, int compute_units);

hipError_t launch_dense_gemm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t stream);

// Canonical compressed activation (vals, idx, scale or null) into the
// workspace regions of ws_layout(M, K, 0).
hipError_t launch_repack(const uint16_t* vals, const uint8_t* idx, const float* scale, int64_t M,
                         int64_t K, void* workspace, hipStream_t stream);

}  // namespace rtl
