// Issue rate of gfx950's bf16 matrix instructions: the measurement behind
// the roofline peaks the benchmark prices its kernels against (a kept
// structured-sparse MAC at the dense MAC rate).  Not part of librtlynx.
//
// Each wavefront issues `iters` rounds of 8 independent instructions of one
// kind (8 accumulator chains, so no instruction waits on the previous one)
// and reads the shader-clock counter (s_memtime) around the loop; a launch of
// one workgroup per CU (each holds 96 KiB of LDS, so no CU takes two) puts 4
// or 8 wavefronts on every CU (1 or 2 per SIMD).
// Cycles per instruction per SIMD = the longest loop of a CU in cycles /
// (iters x 8 x wavefronts per SIMD): independent of the clock the GPU runs at.  Events around the launch
// give the wall time, hence dense-equivalent TFLOP/s and the clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// kinds: 0 v_mfma_f32_16x16x32_bf16, 1 v_mfma_f32_32x32x16_bf16,
//        2 v_smfmac_f32_16x16x64_bf16, 3 v_smfmac_f32_32x32x32_bf16
template <int KIND>
__global__ void __launch_bounds__(512) mfma_rate_kernel(uint64_t* __restrict__ cycles, float* __restrict__ sink,
                                                         int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a;
  bf16x16 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (__bf16)(float)((lane + i) & 7);
#pragma unroll
  for (int i = 0; i < 16; ++i) b[i] = (__bf16)(float)((lane * 3 + i) & 7);
  const bf16x8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7);
  const int idx = 0x4e4e4e4e ^ lane;
  constexpr bool k32 = KIND == 1 || KIND == 3;
  f32x4 acc4[8];
  f32x16 acc16[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc4[j] = (f32x4){0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; ++e) acc16[j][e] = 0.f;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (KIND == 0) acc4[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b8, acc4[j], 0, 0, 0);
      if constexpr (KIND == 1) acc16[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b8, acc16[j], 0, 0, 0);
      if constexpr (KIND == 2) acc4[j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, acc4[j], idx, 0, 0);
      if constexpr (KIND == 3) acc16[j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, acc16[j], idx, 0, 0);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (k32) s += acc16[j][lane & 15];
    else s += acc4[j][lane & 3];
  }
  // 96 KiB of LDS per workgroup: one workgroup per CU (160 KiB), so a
  // launch of one workgroup per CU puts exactly `waves` wavefronts on each.
  __shared__ float hold[24 * 1024];
  hold[threadIdx.x * 48] = s;
  __syncthreads();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = hold[((threadIdx.x + 64) % blockDim.x) * 48];
  if (lane == 0) cycles[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = t1 - t0;
}

}  // namespace

// Launches `blocks` workgroups of 64 * waves threads of instruction kind
// `kind` (0..3) on `stream`; cycles[blocks * waves] and sink[blocks * 64 *
// waves] are device buffers.  Returns the launch's status (0 = success).
extern "C" __attribute__((visibility("default"))) int mb_mfma_rate(int kind, int blocks, int waves, int iters,
                                                                   uint64_t* cycles, float* sink, void* stream) {
  void* args[] = {&cycles, &sink, &iters};
  const void* k = kind == 0   ? reinterpret_cast<const void*>(&mfma_rate_kernel<0>)
                  : kind == 1 ? reinterpret_cast<const void*>(&mfma_rate_kernel<1>)
                  : kind == 2 ? reinterpret_cast<const void*>(&mfma_rate_kernel<2>)
                              : reinterpret_cast<const void*>(&mfma_rate_kernel<3>);
  return (int)hipLaunchKernel(k, dim3(blocks), dim3(64 * waves), args, 0, static_cast<hipStream_t>(stream));
}
