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
#include <type_traits>

#include "gemm_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

template <int KM>
__global__ void __launch_bounds__(kGemmThreads, 1)
sparse_gemm_kernel(const u32x4* __restrict__ xv, const uint32_t* __restrict__ xi,
                   const float* __restrict__ s, const u32x4* __restrict__ tfrag,
                   const uint16_t* __restrict__ w, const uint16_t* __restrict__ lora_b,
                   int64_t M, int64_t N, int64_t K, int64_t r, int64_t kpairs,
                   int64_t rsteps, uint16_t* __restrict__ y) {
  constexpr int kStages = 3;                                   // W ring in LDS, prefetch distance 2
  __shared__ __attribute__((aligned(16))) char lds[kStages][kWTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
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

  // A fragments and index words: two step buffers, filled one step ahead
  // (W runs two steps ahead through the LDS ring).  The workspace keeps the
  // wavefront's 8 row blocks of one k-step in 8 KiB of contiguous memory.
  // Prefetches past the last step re-read the last step (no branch in the
  // loop; the data is never used).
  const int64_t mgroups = (tiles_m * kTileM) / 128;      // 8-block groups in the workspace
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(xv, mgroups * ksteps * 8 * 1024);
  const __amdgpu_buffer_rsrc_t ir = make_rsrc(xi, mgroups * kpairs * 8 * 256);
  const uint32_t a_soff0 = (uint32_t)((mb0 >> 3) * ksteps * 8 * 1024);
  const uint32_t i_soff0 = (uint32_t)((mb0 >> 3) * kpairs * 8 * 256);
  const uint32_t a_voff = 16 * lane, i_voff = 4 * lane;
  u32x4 a_buf[2][kRB];
  uint32_t i_buf[2][kRB];

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, N * K * 2);
  const WTileOffsets wo = w_tile_offsets(K, n0);
  const char* stage_base = &lds[0][0] + 16 * lane + wn * kCB * 2048;

  // Vector-memory operations per thread in one W copy.
  constexpr int kWOps = KM == kAligned8 ? 4 * kWChunksPerThread : kWChunksPerThread;

  auto prefetch_w = [&](int64_t ks, auto stage_c) {
    constexpr int b = decltype(stage_c)::value;
    if constexpr (KM == kAligned8) dma_w_tile_dword(wr, N, K, n0, ks * kTileK, lds[b]);
    else dma_w_tile<KM == kAligned16>(wr, wo, K, ks * kTileK, lds[b]);
  };
  auto prefetch_a = [&](int64_t ks, auto buf_c) {
    constexpr int b = decltype(buf_c)::value;
    const uint32_t so = a_soff0 + (uint32_t)(ks * 8 * 1024);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) a_buf[b][rb] = buf_load16(ar, a_voff, so + rb * 1024);
    const uint32_t si = i_soff0 + (uint32_t)((ks >> 1) * 8 * 256);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      i_buf[b][rb] = __builtin_amdgcn_raw_buffer_load_b32(ir, i_voff + rb * 256, si, 0);
  };

  // One k-step ks (W stage ks % 3, A buffer and index half ks % 2).  Each
  // step issues, in this order, the A loads of step ks + 1 and the W copy of
  // step ks + 2; so at the top of step ks the only operations allowed to be
  // in flight are the W copy of step ks + 1 (kWOps).  The barrier then
  // publishes stage ks % 3 and guarantees that every wave is done with
  // stage (ks + 2) % 3.  The W fragments are read from LDS one column block
  // ahead of the MFMAs.  With the stage a compile-time constant the
  // compiler sees that the copy into stage (ks + 2) % 3 does not alias the
  // reads of stage ks % 3, and does not wait for it.
  auto step = [&](int64_t ks, auto b_c, auto h_c) {
    constexpr int b = decltype(b_c)::value;
    constexpr int h = decltype(h_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kWOps>();
    barrier_no_fence();
    const int64_t ka = ks + 1 < ksteps ? ks + 1 : ksteps - 1;
    const int64_t kw = ks + 2 < ksteps ? ks + 2 : ksteps - 1;
    prefetch_a(ka, std::integral_constant<int, 1 - h>{});
    prefetch_w(kw, std::integral_constant<int, (b + 2) % kStages>{});
    __builtin_amdgcn_sched_barrier(0);
    const char* stage = stage_base + b * kWTileBytes;
    u32x4 b0 = *reinterpret_cast<const u32x4*>(stage);
    u32x4 b1 = *reinterpret_cast<const u32x4*>(stage + 1024);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x16 bf = __builtin_bit_cast(bf16x16, (u32x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
      if (cb + 1 < kCB) {
        b0 = *reinterpret_cast<const u32x4*>(stage + (cb + 1) * 2048);
        b1 = *reinterpret_cast<const u32x4*>(stage + (cb + 1) * 2048 + 1024);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a_buf[h][rb]), bf,
                                                                acc[rb][cb], (int)i_buf[h][rb], 0, h);
    }
  };

  // Prologue: W of steps 0 and 1, A of step 0, in the order the steps assume.
  prefetch_w(0, std::integral_constant<int, 0>{});
  prefetch_a(0, std::integral_constant<int, 0>{});
  prefetch_w(ksteps > 1 ? 1 : 0, std::integral_constant<int, 1>{});
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // ksteps is even; steps run in groups of six so that the stage (ks % 3)
  // and the A buffer / index half (ks % 2) are compile-time constants.
  int64_t ks = 0;
  for (; ks + 6 <= ksteps; ks += 6) {
    step(ks + 0, I0{}, I0{});
    step(ks + 1, I1{}, I1{});
    step(ks + 2, I2{}, I0{});
    step(ks + 3, I0{}, I1{});
    step(ks + 4, I1{}, I0{});
    step(ks + 5, I2{}, I1{});
  }
  if (ks < ksteps) {            // 2 or 4 steps left
    step(ks + 0, I0{}, I0{});
    step(ks + 1, I1{}, I1{});
    if (ks + 2 < ksteps) {
      step(ks + 2, I2{}, I0{});
      step(ks + 3, I0{}, I1{});
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();

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
  // The k loop runs over the padded K (a multiple of 128): full-K mode
  // needs K itself to be one.
  if (K % 128 == 0)
    sparse_gemm_kernel<kFullK><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r,
                                                           L.kp / 128, L.rp / 32, y);
  else if (K % 8 == 0)
    sparse_gemm_kernel<kAligned16><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r,
                                                               L.kp / 128, L.rp / 32, y);
  else
    sparse_gemm_kernel<kAligned8><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r,
                                                              L.kp / 128, L.rp / 32, y);
  return hipGetLastError();
}

}  // namespace rtl
