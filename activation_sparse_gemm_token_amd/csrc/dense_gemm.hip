// rtl_dense_linear: the dense baseline Y = X W^T on gfx950's dense bf16
// matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation, bf16 output.
// This is the denominator of the speedups the RT-Lynx pages quote against
// dense GEMM (qingkeai article, section 05).  It shares the tiling, the W
// ring in LDS, the step structure and the tile order of the structured-
// sparse kernel, so that the two differ only in the A operand and the
// matrix instruction.
//
// The A tile (256 tokens x 64 channels of X per step) goes through LDS in
// the same swizzled row-major layout as W, copied by the same DMA routine,
// in a 2-stage ring next to the 3-stage W ring (96 + 64 KiB of LDS).
#include <type_traits>

#include "gemm_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

// 8 wavefronts (2 x 4), each 128 x 64 = 8 x 4 blocks of 16 x 16: two per
// SIMD, so that one wave's matrix instructions run while the other waits on
// its LDS reads or at the barrier.  (With 4 wavefronts of 128 x 128 the
// matrix cores idled through every such wait and a step took 30 % longer.)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveM = 128, kWaveN = 64;
constexpr int kRB = kWaveM / 16, kCB = kWaveN / 16;

template <int KM>
__global__ void __launch_bounds__(kThreads, 1)
dense_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                  int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y) {
  constexpr int kWStages = 3, kAStages = 2;
  // One LDS block: the W ring, then the A ring; the epilogue reuses all of it.
  constexpr int kLdsBytes = (kWStages + kAStages) * kTileBytes;
  static_assert(store_lds_bytes<kRB, kCB>(kWaves) <= kLdsBytes, "store staging must fit in the rings");
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  char* const lds_w = lds;
  char* const lds_a = lds + kWStages * kTileBytes;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (N + kTileN - 1) / kTileN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t n0 = tn * kTileN;
  const int64_t m0 = tm * kTileM;
  const int64_t ksteps = (K + kTileK - 1) / kTileK;

  f32x4 acc[kRB][kCB];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int j = 0; j < kCB; ++j) acc[i][j] = (f32x4){0, 0, 0, 0};

  // Rows past M / N lie past the end of X / W and read as zeros; channels
  // past K are pointed out of range in the tail modes.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, M * K * 2);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, N * K * 2);
  const WTileOffsets xo = w_tile_offsets<kWaves>(K, m0);
  const WTileOffsets wo = w_tile_offsets<kWaves>(K, n0);
  const uint32_t f0 = frag_lane_offset(0), f1 = frag_lane_offset(1);
  const char* b_base0 = lds_w + wn * kCB * 2048 + f0;
  const char* b_base1 = lds_w + wn * kCB * 2048 + f1;
  const char* a_base0 = lds_a + wm * kRB * 2048 + f0;
  const char* a_base1 = lds_a + wm * kRB * 2048 + f1;
  constexpr int kTileOps = KM == kAligned8 ? 128 / kWaves : 32 / kWaves;

  // Both tile copies are issued as inline-asm DMA blocks: no vector-memory
  // operation of the loop is visible to the compiler, so it inserts no
  // vmcnt waits of its own (it cannot always prove that a copy into one
  // stage does not alias the reads of another) and the explicit waits below
  // are exact.  The K % 8 == 4 mode uses the compiler-visible dword copy.
  auto copy_tile = [&](__amdgpu_buffer_rsrc_t rs, const WTileOffsets& o, int64_t row0, int64_t rows,
                       int64_t ks, char* dst) {
    if constexpr (KM == kAligned8) {
      dma_w_tile_dword<kWaves>(rs, rows, K, row0, ks * kTileK, dst);
    } else {
      const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(dst);
      dma_w_tile_asm<kWaves>(rs, o, K, ks * kTileK, lds_addr, KM == kAligned16);
    }
  };

  // Step ks: W stage ks % 3, A stage ks % 2.  Each step issues the A copy
  // of step ks + 1, then the W copy of step ks + 2, so at its top only the
  // W copy of step ks + 1 may still be in flight.
  auto step = [&](int64_t ks, auto bw_c, auto ba_c) {
    constexpr int bw = decltype(bw_c)::value;
    constexpr int ba = decltype(ba_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kTileOps>();
    barrier_no_fence();
    const int64_t ka = ks + 1 < ksteps ? ks + 1 : ksteps - 1;
    const int64_t kw = ks + 2 < ksteps ? ks + 2 : ksteps - 1;
    copy_tile(xr, xo, m0, M, ka, lds_a + (1 - ba) * kTileBytes);
    copy_tile(wr, wo, n0, N, kw, lds_w + (bw + 2) % kWStages * kTileBytes);
    __builtin_amdgcn_sched_barrier(0);
    const char* bs0 = b_base0 + bw * kTileBytes;
    const char* bs1 = b_base1 + bw * kTileBytes;
    const char* as0 = a_base0 + ba * kTileBytes;
    const char* as1 = a_base1 + ba * kTileBytes;
    bf16x8 af[2][kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      af[0][rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(as0 + rb * 2048));
      af[1][rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(as1 + rb * 2048));
    }
    u32x4 q0 = *reinterpret_cast<const u32x4*>(bs0);
    u32x4 q1 = *reinterpret_cast<const u32x4*>(bs1);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, q0), b1 = __builtin_bit_cast(bf16x8, q1);
      if (cb + 1 < kCB) {
        q0 = *reinterpret_cast<const u32x4*>(bs0 + (cb + 1) * 2048);
        q1 = *reinterpret_cast<const u32x4*>(bs1 + (cb + 1) * 2048);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][rb], b0, acc[rb][cb], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][rb], b1, acc[rb][cb], 0, 0, 0);
    }
  };

  copy_tile(wr, wo, n0, N, 0, lds_w);
  copy_tile(xr, xo, m0, M, 0, lds_a);
  copy_tile(wr, wo, n0, N, ksteps > 1 ? 1 : 0, lds_w + kTileBytes);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int64_t ks = 0;
  for (; ks + 6 <= ksteps; ks += 6) {
    step(ks + 0, I0{}, I0{});
    step(ks + 1, I1{}, I1{});
    step(ks + 2, I2{}, I0{});
    step(ks + 3, I0{}, I1{});
    step(ks + 4, I1{}, I0{});
    step(ks + 5, I2{}, I1{});
  }
  // 0 to 5 steps left (K need not be a multiple of 384).
  if (ks < ksteps) step(ks + 0, I0{}, I0{});
  if (ks + 1 < ksteps) step(ks + 1, I1{}, I1{});
  if (ks + 2 < ksteps) step(ks + 2, I2{}, I0{});
  if (ks + 3 < ksteps) step(ks + 3, I0{}, I1{});
  if (ks + 4 < ksteps) step(ks + 4, I1{}, I0{});
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  barrier_no_fence();                     // every wave is done with the rings

  if (N % 8 == 0) store_tile_via_lds<kRB, kCB>(acc, lds, y, M, N, m0 + wm * kWaveM, n0 + wn * kWaveN);
  else store_acc_bf16<kRB, kCB>(acc, y, M, N, m0 + wm * kWaveM, n0 + wn * kWaveN);
}

}  // namespace

hipError_t launch_dense_gemm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t stream) {
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  const dim3 grid((unsigned)tiles), block(kThreads);
  // 16 x 16 blocks: a form of the same loop on v_mfma_f32_32x32x16_bf16
  // (4 x 2 blocks of 32 x 32 per wavefront) measured 8 % slower (253
  // against 235 us at M = 4096, K = 3072, N = 12288).
  auto* k = K % kTileK == 0 ? &dense_gemm_kernel<kFullK>
            : K % 8 == 0   ? &dense_gemm_kernel<kAligned16>
                           : &dense_gemm_kernel<kAligned8>;
  return launch(k, grid, block, stream, x, w, M, N, K, y);
}

}  // namespace rtl
