// rtl_dense_linear: the dense baseline Y = X W^T on gfx950's dense bf16
// matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation, bf16 output.
// This is the denominator of the speedups the RT-Lynx pages quote against
// dense GEMM (qingkeai article, section 05).  It shares the tiling, the W
// staging and the tile order of the structured-sparse kernel so that the two
// differ only in the A operand and the matrix instruction.
//
// A fragments come straight from X in global memory: lane l takes token
// m0 + l % 16 and channels k + 8 (l / 16) + [0, 8), one 16-byte load.
#include "gemm_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

template <bool ALIGNED16>
__device__ __forceinline__ u32x4 load_a_dense(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                              int64_t m, int64_t k) {
  u32x4 v = (u32x4){0, 0, 0, 0};
  if (m < M) {
    const uint16_t* p = x + m * K + k;
    if constexpr (ALIGNED16) {
      if (k + 8 <= K) v = *reinterpret_cast<const u32x4*>(p);
    } else {
      if (k + 4 <= K) { const u32x2 a = *reinterpret_cast<const u32x2*>(p); v[0] = a[0]; v[1] = a[1]; }
      if (k + 8 <= K) { const u32x2 b = *reinterpret_cast<const u32x2*>(p + 4); v[2] = b[0]; v[3] = b[1]; }
    }
  }
  return v;
}

template <bool ALIGNED16>
__global__ void __launch_bounds__(kGemmThreads, 1)
dense_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                  int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) char lds[2][kWTileBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (N + kTileN - 1) / kTileN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t n0 = tn * kTileN;
  const int64_t m0 = tm * kTileM + wm * kWaveM;
  const int64_t ksteps = (K + kTileK - 1) / kTileK;

  f32x4 acc[kRB][kCB];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int j = 0; j < kCB; ++j) acc[i][j] = (f32x4){0, 0, 0, 0};

  u32x4 a_cur[2][kRB], a_nxt[2][kRB];
  auto load_a = [&](int64_t ks, u32x4 (&a)[2][kRB]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        a[h][rb] = load_a_dense<ALIGNED16>(x, M, K, m0 + 16 * rb + (lane & 15),
                                           ks * kTileK + 32 * h + 8 * (lane >> 4));
  };

  WTileLoader<ALIGNED16> wl;
  wl.issue(w, N, K, n0, 0, lds[0]);
  wl.commit(lds[0]);
  load_a(0, a_cur);

  for (int64_t ks = 0; ks < ksteps; ++ks) {
    wait_vm_all();
    __syncthreads();
    const bool more = ks + 1 < ksteps;
    if (more) {
      wl.issue(w, N, K, n0, (ks + 1) * kTileK, lds[(ks + 1) & 1]);
      load_a(ks + 1, a_nxt);
    }
    const char* stage = lds[ks & 1];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int gcb = wn * kCB + cb;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage + (2 * gcb + h) * 1024 + 16 * lane));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a_cur[h][rb]), b, acc[rb][cb], 0, 0, 0);
      }
    }
    if (more) {
      wl.commit(lds[(ks + 1) & 1]);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) { a_cur[0][rb] = a_nxt[0][rb]; a_cur[1][rb] = a_nxt[1][rb]; }
    }
  }
  store_acc_bf16(acc, y, M, N, m0, n0 + wn * kWaveN);
}

}  // namespace

hipError_t launch_dense_gemm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t stream) {
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  const dim3 grid((unsigned)tiles), block(kGemmThreads);
  if (K % 8 == 0) dense_gemm_kernel<true><<<grid, block, 0, stream>>>(x, w, M, N, K, y);
  else dense_gemm_kernel<false><<<grid, block, 0, stream>>>(x, w, M, N, K, y);
  return hipGetLastError();
}

}  // namespace rtl
