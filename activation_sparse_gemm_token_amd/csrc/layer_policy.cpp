// Selective layer skipping: the per-layer dispatch declared in
// include/rtlynx_layers.h, built on the library's own entry points (the
// dense baseline for skipped layers, the fused layer or a variant for the
// others).
#include "rtlynx.h"
#include "rtlynx_layers.h"

#define RTL_API extern "C" __attribute__((visibility("default")))

namespace rtl {
// rtl_sparse_linear_apply with the choice of the GEMM instance that probes
// the weights into L2 ahead of their copies (rtlynx_api.cpp).
rtl_status apply_impl(const void* workspace, size_t workspace_bytes, const uint16_t* w, const uint16_t* lora_b,
                      int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y, void* hip_stream,
                      bool prefetch_w);
}  // namespace rtl

namespace {

// A sparsification variant as rtl_sparse_linear_prepare_variant accepts it:
// compensation in bits 0-1, LoRA input in bits 2-3 (3 is not a LoRA input).
bool valid_variant(uint32_t v) { return (v & ~0xFu) == 0 && ((v >> 2) & 3u) != 3u; }

// The sizes rtl_sparse_linear_apply adds to those of the prepare: W, Y and
// B, each with the 256 rows past the end its last tile addresses, below
// 2 GiB (the kernels' 32-bit offsets).
bool apply_sizes_ok(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t lim = (int64_t)1 << 31, pad = 256;
  auto ok = [&](int64_t rows, int64_t cols) { return cols == 0 || (cols <= lim / 2 && rows < lim / (2 * cols)); };
  return N < lim && ok(N + pad, K) && ok(M + pad, N) && ok(N + pad, r);
}

}  // namespace

RTL_API rtl_status rtl_layer_linear(const uint32_t* layer_modes, int64_t num_layers, int64_t layer,
                                    const uint16_t* x, const uint16_t* w, const uint16_t* lora_a,
                                    const uint16_t* lora_b, int64_t M, int64_t N, int64_t K, int64_t r,
                                    float lora_scale, uint16_t* y, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  if (num_layers < 0 || layer < 0 || layer >= num_layers) return RTL_ERR_BAD_SHAPE;
  if (layer_modes == nullptr) return RTL_ERR_NULL_POINTER;
  const uint32_t mode = layer_modes[layer] & ~RTL_LAYER_STREAM_W;
  const bool stream_w = (layer_modes[layer] & RTL_LAYER_STREAM_W) != 0;
  if (mode == RTL_LAYER_DENSE) return rtl_dense_linear(x, w, M, N, K, y, hip_stream);
  if (!valid_variant(mode)) return RTL_ERR_BAD_FLAGS;
  if (mode == 0 && !stream_w)
    return rtl_sparse_linear(x, w, lora_a, lora_b, M, N, K, r, lora_scale, y, workspace, workspace_bytes,
                             hip_stream);
  // A variant, or weights streamed: prepare, then apply.  Every argument of
  // the apply is checked before the prepare runs, so an invalid call
  // launches nothing.
  if (N < 0 || !apply_sizes_ok(M, N, K, r)) return RTL_ERR_BAD_SHAPE;
  if (M > 0 && N > 0 && (w == nullptr || y == nullptr || (r > 0 && lora_b == nullptr)))
    return RTL_ERR_NULL_POINTER;
  const size_t need = rtl_sparse_linear_workspace_bytes(M, K, r);
  if (M > 0 && need == 0) return RTL_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return RTL_OK;
  const uintptr_t misaligned = (reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(y) |
                                (r > 0 ? reinterpret_cast<uintptr_t>(lora_b) : 0)) & 15u;
  if (misaligned != 0) return RTL_ERR_MISALIGNED;
  rtl_status st = rtl_sparse_linear_prepare_variant(x, lora_a, M, K, r, lora_scale, mode, workspace,
                                                    workspace_bytes, hip_stream);
  if (st != RTL_OK) return st;
  return rtl::apply_impl(workspace, workspace_bytes, w, lora_b, M, N, K, r, y, hip_stream, stream_w);
}
