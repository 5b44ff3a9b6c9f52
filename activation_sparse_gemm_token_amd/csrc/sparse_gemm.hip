// Structured-sparse GEMM of rtl_sparse_linear with the scale and LoRA-up
// epilogue (qingkeai RT-Lynx article, sections 02 to 04):
//
//   Y[m, n] = bf16( s[m] * sum_k (M*X)[m, k] W[n, k]  +  sum_j (alpha T)[m, j] B[n, j] )
//
// The compressed activation comes from the pre-pass already in the register
// order of v_smfmac_f32_16x16x64_bf16's A operand (lane l: token l % 16, kept
// values of channels 16 (l / 16) + [0, 16), 2-bit positions in a 16-bit
// field; two k-steps share one 32-bit index word, picked with the abid
// operand).  Each wavefront loads its A fragments straight from global
// memory (1 KiB contiguous per fragment) and its W fragments from LDS.  The
// scale is applied to the fp32 accumulators, never folded into a bf16
// operand, and the LoRA-up runs as dense 16x16x32 MFMAs on the hi and lo
// halves of alpha*T.
#include "gemm_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

template <bool ALIGNED16>
__global__ void __launch_bounds__(kGemmThreads, 1)
sparse_gemm_kernel(const u32x4* __restrict__ xv, const uint32_t* __restrict__ xi,
                   const float* __restrict__ s, const u32x4* __restrict__ tfrag,
                   const uint16_t* __restrict__ w, const uint16_t* __restrict__ lora_b,
                   int64_t M, int64_t N, int64_t K, int64_t r, int64_t kpairs,
                   int64_t rsteps, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) char lds[2][kWTileBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (N + kTileN - 1) / kTileN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t n0 = tn * kTileN;
  const int64_t mb0 = (tm * kTileM + wm * kWaveM) / 16;   // first 16-token block of this wavefront
  const int64_t ksteps = 2 * kpairs;

  f32x4 acc[kRB][kCB];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int j = 0; j < kCB; ++j) acc[i][j] = (f32x4){0, 0, 0, 0};

  // A fragments: two step buffers.  Step ks reads buffer ks % 2 while the
  // fragments of step ks + 1 land in the other one.  The workspace keeps the
  // wavefront's 8 row blocks of one k-step in 8 KiB of contiguous memory.
  const u32x4* xa = xv + (mb0 >> 3) * ksteps * 8 * 64 + lane;
  const uint32_t* xa_i = xi + (mb0 >> 3) * kpairs * 8 * 64 + lane;
  u32x4 a_buf[2][kRB];
  uint32_t i_cur[kRB], i_nxt[kRB];
  auto load_a = [&](int64_t ks, u32x4 (&a)[kRB]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) a[rb] = xa[(ks * 8 + rb) * 64];
  };
  auto load_i = [&](int64_t p, uint32_t (&ix)[kRB]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) ix[rb] = xa_i[(p * 8 + rb) * 64];
  };

  WTileLoader<ALIGNED16> wl;
  wl.issue(w, N, K, n0, 0, lds[0]);
  wl.commit(lds[0]);
  load_a(0, a_buf[0]);
  load_i(0, i_cur);

  for (int64_t p = 0; p < kpairs; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t ks = 2 * p + h;
      wait_vm_all();
      __syncthreads();
      const bool more = ks + 1 < ksteps;
      if (more) {
        wl.issue(w, N, K, n0, (ks + 1) * kTileK, lds[(ks + 1) & 1]);
        load_a(ks + 1, a_buf[1 - h]);
        if (h == 1) load_i(p + 1, i_nxt);
      }
      const char* stage = lds[ks & 1];
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int gcb = wn * kCB + cb;
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(stage + (2 * gcb) * 1024 + 16 * lane);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(stage + (2 * gcb + 1) * 1024 + 16 * lane);
        const bf16x16 b = __builtin_bit_cast(bf16x16, (u32x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if (h == 0)
            acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a_buf[0][rb]), b, acc[rb][cb], (int)i_cur[rb], 0, 0);
          else
            acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a_buf[1][rb]), b, acc[rb][cb], (int)i_cur[rb], 0, 1);
        }
      }
      if (more) wl.commit(lds[(ks + 1) & 1]);
    }
    if (p + 1 < kpairs) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) i_cur[rb] = i_nxt[rb];
    }
  }

  // Epilogue 1: per-token compensation scale on the fp32 accumulators.
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int64_t mb = mb0 + rb;
    const f32x4 sv = *reinterpret_cast<const f32x4*>(s + mb * 16 + 4 * (lane >> 4));
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rb][cb][i] *= sv[i];
  }

  // Epilogue 2: LoRA-up, (alpha T)_hi B^T + (alpha T)_lo B^T on dense MFMAs.
  if (r > 0) {
    for (int64_t rs = 0; rs < rsteps; ++rs) {
      bf16x8 bfr[kCB];
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int64_t n = n0 + wn * kWaveN + 16 * cb + (lane & 15);
        const int64_t j = 32 * rs + 8 * (lane >> 4);
        u32x4 v = (u32x4){0, 0, 0, 0};
        if (n < N) {
          const uint16_t* pb = lora_b + n * r + j;
          if (r % 8 == 0) {
            if (j + 8 <= r) v = *reinterpret_cast<const u32x4*>(pb);
          } else {
            uint16_t e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) e[t] = (j + t < r) ? pb[t] : (uint16_t)0;
            v = (u32x4){e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                        e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
          }
        }
        bfr[cb] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int64_t mb = mb0 + rb;
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          const bf16x8 ta = __builtin_bit_cast(bf16x8, tfrag[((mb * rsteps + rs) * 2 + hl) * 64 + lane]);
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta, bfr[cb], acc[rb][cb], 0, 0, 0);
        }
      }
    }
  }

  store_acc_bf16(acc, y, M, N, tm * kTileM + wm * kWaveM, n0 + wn * kWaveN);
}

}  // namespace

hipError_t launch_sparse_gemm(const void* workspace, const uint16_t* w, const uint16_t* lora_b,
                              int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y,
                              hipStream_t stream) {
  const WsLayout L = ws_layout(M, K, r);
  const char* ws = static_cast<const char*>(workspace);
  const u32x4* xv = reinterpret_cast<const u32x4*>(ws + L.off_xv);
  const uint32_t* xi = reinterpret_cast<const uint32_t*>(ws + L.off_xi);
  const float* s = reinterpret_cast<const float*>(ws + L.off_s);
  const u32x4* t = reinterpret_cast<const u32x4*>(ws + L.off_t);
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  const dim3 grid((unsigned)tiles), block(kGemmThreads);
  if (K % 8 == 0)
    sparse_gemm_kernel<true><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r,
                                                         L.kp / 128, L.rp / 32, y);
  else
    sparse_gemm_kernel<false><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r,
                                                          L.kp / 128, L.rp / 32, y);
  return hipGetLastError();
}

}  // namespace rtl
