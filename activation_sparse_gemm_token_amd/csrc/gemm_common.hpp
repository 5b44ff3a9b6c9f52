// Pieces shared by the structured-sparse and the dense GEMM kernels.
//
// Both kernels compute a 256 x 256 output tile per workgroup of 4
// wavefronts (2 x 2, each 128 x 128 = 8 x 8 blocks of 16 x 16) and stream
// the weight through LDS in 64-deep k-steps, double-buffered.  The LDS copy
// of a W tile is stored in matrix-core operand order: for every 16-column
// block and every 32-channel half of the k-step, 64 lanes x 16 bytes, where
// lane l holds column l % 16, channels 8 (l / 16) + [0, 8).  That is the B
// operand of v_mfma_f32_16x16x32_bf16 for one half, and the two halves
// together form the B operand of v_smfmac_f32_16x16x64_bf16, so each
// wavefront reads its operands with lane-contiguous 16-byte LDS reads.
#pragma once

#include "rtl_common.hpp"

namespace rtl {

constexpr int kTileM = 256, kTileN = 256, kTileK = 64;
constexpr int kGemmThreads = 256;
constexpr int kWaveM = 128, kWaveN = 128;
constexpr int kRB = kWaveM / 16, kCB = kWaveN / 16;          // 8 x 8 blocks per wavefront
constexpr int kWTileBytes = kTileN * kTileK * 2;             // 32 KiB per stage
constexpr int kWChunksPerThread = kWTileBytes / 16 / kGemmThreads;   // 8

// W-tile copy.  Thread (wave v, lane l) moves chunk i: 16-column block
// cb = 4 v + i / 2, half h = i % 2, column n0 + 16 cb + l % 16, channels
// k0 + 32 h + 8 (l / 16) + [0, 8), to LDS byte offset (2 cb + h) * 1024 + 16 l.
// Columns past N read row N - 1 (their results are never stored).  Channels
// past K read channel 0 of the same row: finite values that meet zeros in
// the A operand.
//
// With 16-byte aligned rows (K % 8 == 0) the copy is a direct global -> LDS
// load (global_load_lds_dwordx4), which writes lane l's 16 bytes to
// base + 16 l and needs no registers; the caller waits on vmcnt before the
// barrier that publishes the stage.  Otherwise rows are 8-byte aligned and the
// copy goes through registers in 8-byte halves.
__device__ __forceinline__ const uint16_t* w_chunk_ptr(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                       int64_t n0, int64_t k0, int i, int64_t& k) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = 4 * wave + i / 2, h = i % 2;
  int64_t n = n0 + 16 * cb + (lane & 15);
  n = n < N ? n : N - 1;
  k = k0 + 32 * h + 8 * (lane >> 4);
  return w + n * K;
}

__device__ __forceinline__ void load_w_tile_direct(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                   int64_t n0, int64_t k0, char* lds_stage) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kWChunksPerThread; ++i) {
    int64_t k;
    const uint16_t* row = w_chunk_ptr(w, N, K, n0, k0, i, k);
    const uint16_t* src = row + (k + 8 <= K ? k : 0);
    char* dst = lds_stage + (2 * (4 * wave + i / 2) + i % 2) * 1024;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
  }
}

__device__ __forceinline__ void load_w_tile_regs(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                 int64_t n0, int64_t k0, u32x4 (&st)[kWChunksPerThread]) {
#pragma unroll
  for (int i = 0; i < kWChunksPerThread; ++i) {
    int64_t k;
    const uint16_t* p = w_chunk_ptr(w, N, K, n0, k0, i, k) + k;
    u32x4 v = (u32x4){0, 0, 0, 0};
    if (k + 4 <= K) { const u32x2 a = *reinterpret_cast<const u32x2*>(p); v[0] = a[0]; v[1] = a[1]; }
    if (k + 8 <= K) { const u32x2 b = *reinterpret_cast<const u32x2*>(p + 4); v[2] = b[0]; v[3] = b[1]; }
    st[i] = v;
  }
}

__device__ __forceinline__ void store_w_tile(char* lds_stage, const u32x4 (&st)[kWChunksPerThread]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kWChunksPerThread; ++i) {
    const int cb = 4 * wave + i / 2, h = i % 2;
    *reinterpret_cast<u32x4*>(lds_stage + (2 * cb + h) * 1024 + 16 * lane) = st[i];
  }
}

// Issues the copy of one W tile into an LDS stage.  In the register path the
// LDS write is deferred to commit_w_tile so that the global loads overlap the
// matrix work of the current stage.
template <bool ALIGNED16>
struct WTileLoader {
  u32x4 st[ALIGNED16 ? 1 : kWChunksPerThread];
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                        int64_t n0, int64_t k0, char* lds_stage) {
    if constexpr (ALIGNED16) load_w_tile_direct(w, N, K, n0, k0, lds_stage);
    else load_w_tile_regs(w, N, K, n0, k0, st);
  }
  __device__ __forceinline__ void commit(char* lds_stage) {
    if constexpr (!ALIGNED16) store_w_tile(lds_stage, st);
  }
};

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Tile order: tiles are taken in column panels of kGroupM tile rows so that
// workgroups running together share W panels in L2.
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  const int64_t id = blockIdx.x;
  const int64_t per_group = (int64_t)kGroupM * tiles_n;
  const int64_t g = id / per_group;
  const int64_t first_m = g * kGroupM;
  const int64_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int64_t in = id - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Stores a wavefront's 128 x 128 fp32 accumulators as bf16.
__device__ __forceinline__ void store_acc_bf16(const f32x4 (&acc)[kRB][kCB], uint16_t* __restrict__ y,
                                               int64_t M, int64_t N, int64_t m0, int64_t n0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int64_t n = n0 + 16 * cb + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 16 * rb + 4 * (lane >> 4) + i;
        if (m < M && n < N) y[m * N + n] = (uint16_t)f32_to_bf16_rne(acc[rb][cb][i]);
      }
    }
  }
}

}  // namespace rtl
