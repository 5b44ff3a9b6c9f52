// Host side of librtlynx: argument validation, device checks and launches
// behind the C ABI declared in include/rtlynx.h.
//
// Validation is pure arithmetic on the arguments and runs before any HIP
// call, so an invalid call touches neither the device nor the runtime's
// error state.  The only process-wide state is a per-device cache of the
// "is this a gfx950" answer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "rtl_common.hpp"
#include "rtl_kernels.hpp"
#include "rtlynx.h"

#define RTL_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kVersion = 10000;            // 1.0.0
constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int kMaxDevices = 64;

std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];       // compute units of a known device

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dims_ok(int64_t M, int64_t K) {
  return M >= 0 && K >= 4 && K % 4 == 0 && M < kMaxDim && K < kMaxDim;
}

// The GEMM kernels address each tensor through a buffer resource with a
// 32-bit size and 32-bit offsets.
constexpr int64_t kMaxBytes = (int64_t)1 << 31;

bool bytes_ok(int64_t rows, int64_t cols, int64_t elem) {
  return rows == 0 || cols == 0 || (cols <= kMaxBytes / elem && rows < kMaxBytes / (cols * elem));
}

// Every tensor and workspace region of a linear-layer call below 2 GiB,
// counting the up to 255 rows past the end that the last 256-row tile of
// X, W and Y addresses (they read as zeros / are not written).
bool layer_sizes_ok(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t pad = 256;
  if (!bytes_ok(M + pad, K, 2) || !bytes_ok(N + pad, K, 2) || !bytes_ok(M + pad, N, 2) ||
      !bytes_ok(r, K, 2) || !bytes_ok(N + pad, r, 2))
    return false;
  if (M == 0) return true;
  const rtl::WsLayout L = rtl::ws_layout(M, K, r);
  return bytes_ok(L.mp, L.kp, 1) && bytes_ok(L.mp, L.rp, 4);
}

// Checks that a gfx950 device is current and that `stream` (NULL: the null
// stream) belongs to it; sets *cus to its CU count.
rtl_status check_device(hipStream_t stream, int* cus = nullptr) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return RTL_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return RTL_ERR_NO_DEVICE;
  }
  if (stream != nullptr) {
    // The kernels run on the stream's device with the current device's
    // launch parameters (and, without a workspace, its scratch array).
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return RTL_ERR_HIP;
    }
    if (sdev != dev) return RTL_ERR_STREAM_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return RTL_ERR_UNSUPPORTED_ARCH;
  int known = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return RTL_ERR_HIP;
    }
    known = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_ok[dev].store(known, std::memory_order_relaxed);
  }
  if (cus != nullptr) *cus = g_cus[dev].load(std::memory_order_relaxed);
  return known == 1 ? RTL_OK : RTL_ERR_UNSUPPORTED_ARCH;
}

rtl_status from_hip(hipError_t e) { return e == hipSuccess ? RTL_OK : RTL_ERR_HIP; }

// Scratch of rtl_sparse_linear_noalloc: the workspace of the layer, held in
// a device array of fixed size that each GPU running the library keeps
// until the process ends.  Host code never uses the array's name as an
// address (on the host it names a stand-in, not device memory): the device
// address is read once per device with hipGetSymbolAddress, with that
// device current, and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[RTL_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device `dev`, or nullptr if
// the runtime cannot provide it.
void* scratch_address(int dev) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

RTL_API rtl_status rtl_sparsify_2of4(const uint16_t* x, int64_t M, int64_t K, uint16_t* vals,
                                     uint8_t* idx, float* scale, uint32_t flags, void* hip_stream) {
  if (!dims_ok(M, K)) return RTL_ERR_BAD_SHAPE;
  if ((flags & ~RTL_FOLD_SCALE) != 0) return RTL_ERR_BAD_FLAGS;
  if (M == 0) return RTL_OK;
  if (x == nullptr || vals == nullptr || idx == nullptr) return RTL_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(vals) || !aligned16(idx) || (scale != nullptr && !aligned16(scale)))
    return RTL_ERR_MISALIGNED;
  int cus = 0;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream), &cus);
  if (d != RTL_OK) return d;
  return from_hip(rtl::launch_sparsify_2of4(x, M, K, vals, idx, scale, (flags & RTL_FOLD_SCALE) != 0, cus,
                                            static_cast<hipStream_t>(hip_stream)));
}

RTL_API size_t rtl_sparse_linear_workspace_bytes(int64_t M, int64_t K, int64_t r) {
  if (!dims_ok(M, K) || r < 0 || r > RTL_MAX_LORA_RANK || !layer_sizes_ok(M, 0, K, r)) return 0;
  if (M == 0) return 0;
  return rtl::ws_layout(M, K, r).total;
}

RTL_API rtl_status rtl_sparse_linear_prepare(const uint16_t* x, const uint16_t* lora_a, int64_t M,
                                             int64_t K, int64_t r, float lora_scale, void* workspace,
                                             size_t workspace_bytes, void* hip_stream) {
  if (!dims_ok(M, K) || r < 0 || r > RTL_MAX_LORA_RANK) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, 0, K, r)) return RTL_ERR_BAD_SHAPE;
  if (M == 0) return RTL_OK;
  if (x == nullptr) return RTL_ERR_NULL_POINTER;
  if (r > 0 && lora_a == nullptr) return RTL_ERR_NULL_POINTER;
  if (!aligned16(x) || (r > 0 && !aligned16(lora_a))) return RTL_ERR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < rtl::ws_layout(M, K, r).total) return RTL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RTL_ERR_MISALIGNED;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream));
  if (d != RTL_OK) return d;
  return from_hip(rtl::launch_prepass(x, r > 0 ? lora_a : nullptr, M, K, r, lora_scale, workspace,
                                      static_cast<hipStream_t>(hip_stream)));
}

RTL_API rtl_status rtl_sparse_linear_prepare_variant(const uint16_t* x, const uint16_t* lora_a, int64_t M,
                                                     int64_t K, int64_t r, float lora_scale, uint32_t variant,
                                                     void* workspace, size_t workspace_bytes, void* hip_stream) {
  const uint32_t comp = variant & 3u, lora = (variant >> 2) & 3u;
  if ((variant & ~0xFu) != 0 || lora == 3u) return RTL_ERR_BAD_FLAGS;
  if (!dims_ok(M, K) || r < 0 || r > RTL_MAX_LORA_RANK) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, 0, K, r)) return RTL_ERR_BAD_SHAPE;
  if (M == 0) return RTL_OK;
  if (x == nullptr) return RTL_ERR_NULL_POINTER;
  if (r > 0 && lora_a == nullptr) return RTL_ERR_NULL_POINTER;
  if (!aligned16(x) || (r > 0 && !aligned16(lora_a))) return RTL_ERR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < rtl::ws_layout(M, K, r).total) return RTL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RTL_ERR_MISALIGNED;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream));
  if (d != RTL_OK) return d;
  return from_hip(rtl::launch_prepass(x, r > 0 ? lora_a : nullptr, M, K, r, lora_scale, workspace,
                                      static_cast<hipStream_t>(hip_stream), (int)comp, (int)lora));
}

namespace rtl {

rtl_status apply_impl(const void* workspace, size_t workspace_bytes, const uint16_t* w, const uint16_t* lora_b,
                      int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y, void* hip_stream,
                      bool prefetch_w) {
  if (!dims_ok(M, K) || N < 0 || N >= kMaxDim || r < 0 || r > RTL_MAX_LORA_RANK) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, N, K, r)) return RTL_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return RTL_OK;
  if (w == nullptr || y == nullptr) return RTL_ERR_NULL_POINTER;
  if (r > 0 && lora_b == nullptr) return RTL_ERR_NULL_POINTER;
  if (!aligned16(w) || !aligned16(y) || (r > 0 && !aligned16(lora_b))) return RTL_ERR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < rtl::ws_layout(M, K, r).total) return RTL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RTL_ERR_MISALIGNED;
  int cus = 0;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream), &cus);
  if (d != RTL_OK) return d;
  return from_hip(rtl::launch_sparse_gemm(workspace, w, r > 0 ? lora_b : nullptr, M, N, K, r, y, cus,
                                          static_cast<hipStream_t>(hip_stream), 0, prefetch_w));
}

}  // namespace rtl

RTL_API rtl_status rtl_sparse_linear_apply(const void* workspace, size_t workspace_bytes,
                                           const uint16_t* w, const uint16_t* lora_b, int64_t M,
                                           int64_t N, int64_t K, int64_t r, uint16_t* y,
                                           void* hip_stream) {
  return rtl::apply_impl(workspace, workspace_bytes, w, lora_b, M, N, K, r, y, hip_stream, false);
}

RTL_API rtl_status rtl_sparse_linear(const uint16_t* x, const uint16_t* w, const uint16_t* lora_a,
                                     const uint16_t* lora_b, int64_t M, int64_t N, int64_t K,
                                     int64_t r, float lora_scale, uint16_t* y, void* workspace,
                                     size_t workspace_bytes, void* hip_stream) {
  if (!dims_ok(M, K) || N < 0 || N >= kMaxDim || r < 0 || r > RTL_MAX_LORA_RANK) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, N, K, r)) return RTL_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return RTL_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return RTL_ERR_NULL_POINTER;
  if (r > 0 && (lora_a == nullptr || lora_b == nullptr)) return RTL_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return RTL_ERR_MISALIGNED;
  if (r > 0 && (!aligned16(lora_a) || !aligned16(lora_b))) return RTL_ERR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < rtl::ws_layout(M, K, r).total) return RTL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RTL_ERR_MISALIGNED;
  int cus = 0;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream), &cus);
  if (d != RTL_OK) return d;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (rtl::launch_prepass(x, r > 0 ? lora_a : nullptr, M, K, r, lora_scale, workspace, stream) != hipSuccess)
    return RTL_ERR_HIP;
  return from_hip(rtl::launch_sparse_gemm(workspace, w, r > 0 ? lora_b : nullptr, M, N, K, r, y, cus, stream));
}

RTL_API rtl_status rtl_sparse_linear_noalloc(const uint16_t* x, const uint16_t* w, const uint16_t* lora_a,
                                             const uint16_t* lora_b, int64_t M, int64_t N, int64_t K, int64_t r,
                                             float lora_scale, uint16_t* y, void* hip_stream) {
  if (!dims_ok(M, K) || N < 0 || N >= kMaxDim || r < 0 || r > RTL_MAX_LORA_RANK) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, N, K, r)) return RTL_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return RTL_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return RTL_ERR_NULL_POINTER;
  if (r > 0 && (lora_a == nullptr || lora_b == nullptr)) return RTL_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return RTL_ERR_MISALIGNED;
  if (r > 0 && (!aligned16(lora_a) || !aligned16(lora_b))) return RTL_ERR_MISALIGNED;
  if (rtl::ws_layout(M, K, r).total > (size_t)RTL_NOALLOC_SCRATCH_BYTES) return RTL_ERR_WORKSPACE;
  int cus = 0;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream), &cus);
  if (d != RTL_OK) return d;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RTL_ERR_NO_DEVICE;
  void* ws = scratch_address(dev);
  if (ws == nullptr) return RTL_ERR_HIP;
  // The pre-pass writes every workspace region the GEMM reads (all padded
  // rows, k-steps and rank columns), so nothing needs clearing first.
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (rtl::launch_prepass(x, r > 0 ? lora_a : nullptr, M, K, r, lora_scale, ws, stream) != hipSuccess)
    return RTL_ERR_HIP;
  return from_hip(rtl::launch_sparse_gemm(ws, w, r > 0 ? lora_b : nullptr, M, N, K, r, y, cus, stream));
}

RTL_API rtl_status rtl_sparse_linear_compressed(const uint16_t* vals, const uint8_t* idx, const float* scale,
                                                const uint16_t* w, int64_t M, int64_t N, int64_t K, uint16_t* y,
                                                void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!dims_ok(M, K) || N < 0 || N >= kMaxDim) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, N, K, 0)) return RTL_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return RTL_OK;
  if (vals == nullptr || idx == nullptr || w == nullptr || y == nullptr) return RTL_ERR_NULL_POINTER;
  if (!aligned16(vals) || !aligned16(idx) || !aligned16(w) || !aligned16(y) ||
      (scale != nullptr && !aligned16(scale)))
    return RTL_ERR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < rtl::ws_layout(M, K, 0).total) return RTL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RTL_ERR_MISALIGNED;
  int cus = 0;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream), &cus);
  if (d != RTL_OK) return d;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = rtl::launch_repack(vals, idx, scale, M, K, workspace, stream);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(rtl::launch_sparse_gemm(workspace, w, nullptr, M, N, K, 0, y, cus, stream));
}

RTL_API rtl_status rtl_dense_linear(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                    int64_t K, uint16_t* y, void* hip_stream) {
  if (!dims_ok(M, K) || N < 0 || N >= kMaxDim) return RTL_ERR_BAD_SHAPE;
  if (!layer_sizes_ok(M, N, K, 0)) return RTL_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return RTL_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return RTL_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return RTL_ERR_MISALIGNED;
  const rtl_status d = check_device(static_cast<hipStream_t>(hip_stream));
  if (d != RTL_OK) return d;
  return from_hip(rtl::launch_dense_gemm(x, w, M, N, K, y, static_cast<hipStream_t>(hip_stream)));
}

RTL_API const char* rtl_status_string(rtl_status s) {
  switch (s) {
    case RTL_OK: return "ok";
    case RTL_ERR_NULL_POINTER: return "a required pointer is NULL";
    case RTL_ERR_BAD_SHAPE: return "invalid shape (sizes must be >= 0, K >= 4 and K % 4 == 0, r <= RTL_MAX_LORA_RANK, every tensor below 2 GiB)";
    case RTL_ERR_MISALIGNED: return "a base pointer is not 16-byte aligned";
    case RTL_ERR_WORKSPACE: return "workspace missing or smaller than rtl_sparse_linear_workspace_bytes()";
    case RTL_ERR_NO_DEVICE: return "no HIP device is visible";
    case RTL_ERR_UNSUPPORTED_ARCH: return "the current device is not gfx950 (MI355X)";
    case RTL_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case RTL_ERR_BAD_FLAGS: return "unknown flag bits";
    case RTL_ERR_STREAM_DEVICE: return "hip_stream belongs to a device other than the current one";
  }
  return "unknown status";
}

RTL_API int rtl_version(void) { return kVersion; }
