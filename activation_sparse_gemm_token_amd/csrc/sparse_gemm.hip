// Structured-sparse GEMM of rtl_sparse_linear with the scale and LoRA-up
// epilogue (qingkeai RT-Lynx article, sections 02 to 04):
//
//   Y[m, n] = bf16( s[m] * sum_k (M*X)[m, k] W[n, k]  +  sum_j (alpha T)[m, j] B[n, j] )
//
// computed as Y = bf16( s * ( S(X) W^T + (alpha T / s) B^T ) ).
//
// The compressed activation comes from the pre-pass already in the register
// order of v_smfmac_f32_16x16x64_bf16's A operand (lane l: token l % 16, kept
// values of channels 16 (l / 16) + [0, 16), 2-bit positions in a 16-bit
// field; the fields of two 16-token blocks share one 32-bit word, picked
// with the abid operand).  Every operand reaches LDS by DMA through one
// 3-stage ring: first the K/64 structured-sparse k-steps, then r/32 LoRA
// steps that run dense 16x16x32 MFMAs on the hi and lo halves of
// alpha T / s (pre-pass) against B, into the same accumulators.  The scale
// is applied once to the fp32 accumulators, never folded into a bf16
// operand, and the tile leaves through LDS as coalesced 16-byte stores.
#include "gemm_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

// Per k-step LDS stage: the W tile (32 KiB), the workgroup's 256 rows of
// compressed A (16 x 1 KiB fragments) and their position fields (2 x 1 KiB).
// A LoRA step puts the 256 rows of alpha T / s (16 blocks x hi, lo x 1 KiB)
// where W goes and the 256 columns of B (16 x 1 KiB) where A goes.
constexpr int kAStageOff = kWTileBytes;
constexpr int kIStageOff = kWTileBytes + 16 * 1024;
constexpr int kStageBytes = kWTileBytes + 18 * 1024;
constexpr int kStages = 3;                                   // prefetch distance 2
constexpr int kScaleOff = kStages * kStageBytes;             // 256 per-token scales
constexpr int kLdsBytes = kScaleOff + 1024;
static_assert(kStoreLdsBytes <= kScaleOff, "store staging must not reach the scales");

// Copies the compressed A operand of one k-step into an LDS stage: thread
// (wave v, i) moves fragment c = 4 v + i (16-token block c % 8 of group
// c / 8) with one buffer_load_dwordx4 ... lds, and 256 bytes of the position
// fields with each of two buffer_load_dword ... lds (parts 2v, 2v + 1 of the
// two groups' 2 KiB).  Same rules as dma_w_tile_asm: no output registers,
// M0 saved and restored, no SCC write.  6 vector-memory operations.
__device__ __forceinline__ void dma_a_tile_asm(__amdgpu_buffer_rsrc_t ar, __amdgpu_buffer_rsrc_t ir,
                                               uint32_t a_group0, uint32_t i_group0, uint32_t a_gstride,
                                               uint32_t i_gstride, int64_t ks, uint32_t lds_stage_addr) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // fragments 4v .. 4v+3 all lie in group v / 2, blocks 4 (v % 2) .. +3
  const uint32_t g = wave >> 1;
  const uint32_t a_so = __builtin_amdgcn_readfirstlane(a_group0 + g * a_gstride + (uint32_t)ks * 8192u +
                                                       (wave & 1u) * 4096u);
  const uint32_t la = __builtin_amdgcn_readfirstlane(lds_stage_addr + kAStageOff + wave * 4096u);
  // position parts 2v, 2v+1: group v / 2, bytes 512 (v % 2) .. +512
  const uint32_t i_so = __builtin_amdgcn_readfirstlane(i_group0 + g * i_gstride + (uint32_t)ks * 1024u +
                                                       (wave & 1u) * 512u);
  const uint32_t li = __builtin_amdgcn_readfirstlane(lds_stage_addr + kIStageOff + wave * 512u);
  const uint32_t va = 16u * lane, vi = 4u * lane;
  uint32_t saved;
  // The instruction offset of a buffer ... lds load is added to the LDS
  // address too, so every offset is carried by the scalar offset operand.
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[la0]\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso0] offen lds\n\t"
      "s_mov_b32 m0, %[la1]\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso1] offen lds\n\t"
      "s_mov_b32 m0, %[la2]\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso2] offen lds\n\t"
      "s_mov_b32 m0, %[la3]\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso3] offen lds\n\t"
      "s_mov_b32 m0, %[li0]\n\t"
      "buffer_load_dword %[vi], %[ir], %[iso0] offen lds\n\t"
      "s_mov_b32 m0, %[li1]\n\t"
      "buffer_load_dword %[vi], %[ir], %[iso1] offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [va] "v"(va), [vi] "v"(vi), [ar] "s"(ar), [ir] "s"(ir),
        [aso0] "s"(a_so), [aso1] "s"(a_so + 1024u), [aso2] "s"(a_so + 2048u), [aso3] "s"(a_so + 3072u),
        [iso0] "s"(i_so), [iso1] "s"(i_so + 256u),
        [la0] "s"(la), [la1] "s"(la + 1024u), [la2] "s"(la + 2048u), [la3] "s"(la + 3072u),
        [li0] "s"(li), [li1] "s"(li + 256u)
      : "memory");
  (void)saved;
}

// Copies the operands of LoRA step rs into an LDS stage: thread (wave v,
// i < 8) moves 1 KiB of alpha T / s (16-token block 4 v + i / 2, half i % 2)
// and thread (v, i < 4) 1 KiB of B (columns n0 + 16 (4 v + i) + [0, 16),
// ranks 32 rs + 8 (l / 16) + [0, 8)).  B rows past N and rank chunks past r
// carry their whole offset in the VGPR operand and read as zeros.  The last
// two B copies are issued twice, so that a LoRA step issues as many
// vector-memory operations (14) as a k-step and the waits stay uniform.
__device__ __forceinline__ void dma_lora_tile_asm(__amdgpu_buffer_rsrc_t tr, __amdgpu_buffer_rsrc_t br,
                                                  uint32_t t_block0, int64_t rsteps, int64_t rs,
                                                  int64_t N, int64_t r, int64_t n0, uint32_t lds_stage_addr) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t blk = __builtin_amdgcn_readfirstlane((uint32_t)(rsteps * 2048));
  const uint32_t t_so = __builtin_amdgcn_readfirstlane(t_block0 + 4u * wave * blk + (uint32_t)rs * 2048u);
  const uint32_t lt = __builtin_amdgcn_readfirstlane(lds_stage_addr + wave * 8192u);
  const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_stage_addr + kAStageOff + wave * 4096u);
  const uint32_t vt = 16u * lane;
  const int64_t j = 32 * rs + 8 * (lane >> 4);
  uint32_t vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + 16 * (4 * (int64_t)wave + i) + (lane & 15);
    vb[i] = (n < N && j + 8 <= r) ? (uint32_t)((n * r + j) * 2) : kOobOffset;
  }
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lt0]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts0] offen lds\n\t"
      "s_mov_b32 m0, %[lt1]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts1] offen lds\n\t"
      "s_mov_b32 m0, %[lt2]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts2] offen lds\n\t"
      "s_mov_b32 m0, %[lt3]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts3] offen lds\n\t"
      "s_mov_b32 m0, %[lt4]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts4] offen lds\n\t"
      "s_mov_b32 m0, %[lt5]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts5] offen lds\n\t"
      "s_mov_b32 m0, %[lt6]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts6] offen lds\n\t"
      "s_mov_b32 m0, %[lt7]\n\t"
      "buffer_load_dwordx4 %[vt], %[tr], %[ts7] offen lds\n\t"
      "s_mov_b32 m0, %[lb0]\n\t"
      "buffer_load_dwordx4 %[vb0], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb1]\n\t"
      "buffer_load_dwordx4 %[vb1], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb2]\n\t"
      "buffer_load_dwordx4 %[vb2], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb3]\n\t"
      "buffer_load_dwordx4 %[vb3], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb2]\n\t"
      "buffer_load_dwordx4 %[vb2], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb3]\n\t"
      "buffer_load_dwordx4 %[vb3], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [vt] "v"(vt), [vb0] "v"(vb[0]), [vb1] "v"(vb[1]), [vb2] "v"(vb[2]), [vb3] "v"(vb[3]),
        [tr] "s"(tr), [br] "s"(br),
        [ts0] "s"(t_so), [ts1] "s"(t_so + 1024u), [ts2] "s"(t_so + blk), [ts3] "s"(t_so + blk + 1024u),
        [ts4] "s"(t_so + 2u * blk), [ts5] "s"(t_so + 2u * blk + 1024u), [ts6] "s"(t_so + 3u * blk),
        [ts7] "s"(t_so + 3u * blk + 1024u),
        [lt0] "s"(lt), [lt1] "s"(lt + 1024u), [lt2] "s"(lt + 2048u), [lt3] "s"(lt + 3072u),
        [lt4] "s"(lt + 4096u), [lt5] "s"(lt + 5120u), [lt6] "s"(lt + 6144u), [lt7] "s"(lt + 7168u),
        [lb0] "s"(lb), [lb1] "s"(lb + 1024u), [lb2] "s"(lb + 2048u), [lb3] "s"(lb + 3072u)
      : "memory");
  (void)saved;
}

// Copies the workgroup's 256 per-token scales into LDS (one dword DMA per
// thread).  1 vector-memory operation.
__device__ __forceinline__ void dma_scale_asm(__amdgpu_buffer_rsrc_t sr, uint32_t row0_bytes,
                                              uint32_t lds_scale_addr) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t so = __builtin_amdgcn_readfirstlane(row0_bytes + 256u * wave);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(lds_scale_addr + 256u * wave);
  const uint32_t v = 4u * lane;
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[ls]\n\t"
      "buffer_load_dword %[v], %[sr], %[so] offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [v] "v"(v), [sr] "s"(sr), [so] "s"(so), [ls] "s"(ls)
      : "memory");
  (void)saved;
}

// RING: the LoRA-up runs as extra steps of the LDS ring (r % 8 == 0 and
// 16-byte W rows).  Otherwise it runs after the k loop from global memory
// (odd ranks, K % 8 == 4: shapes outside the fast path).
template <int KM, bool RING>
__global__ void __launch_bounds__(kGemmThreads, 1)
sparse_gemm_kernel(const u32x4* __restrict__ xv, const uint16_t* __restrict__ xi,
                   const float* __restrict__ s, const u32x4* __restrict__ tfrag,
                   const uint16_t* __restrict__ w, const uint16_t* __restrict__ lora_b,
                   int64_t M, int64_t N, int64_t K, int64_t r, int64_t kpairs,
                   int64_t rsteps, uint16_t* __restrict__ y) {
  static_assert(!RING || KM != kAligned8, "the ring's uniform waits need 14 operations per step");
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (N + kTileN - 1) / kTileN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t n0 = tn * kTileN;
  const int64_t mb0 = (tm * kTileM + wm * kWaveM) / 16;   // first 16-token block of this wavefront
  const int64_t ksteps = 2 * kpairs;
  const int64_t lsteps = RING && r > 0 ? rsteps : 0;
  const int64_t total = ksteps + lsteps;

  f32x4 acc[kRB][kCB];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int j = 0; j < kCB; ++j) acc[i][j] = (f32x4){0, 0, 0, 0};

  // Every operand of the loop arrives by DMA into a 3-stage LDS ring, two
  // steps ahead; nothing in the loop is a compiler-visible memory load, so
  // the explicit vmcnt waits are exact.
  const int64_t mgroups = (tiles_m * kTileM) / 128;      // 8-block groups in the workspace
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(xv, mgroups * ksteps * 8192);
  const __amdgpu_buffer_rsrc_t ir = make_rsrc(xi, mgroups * ksteps * 1024);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, N * K * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, tiles_m * kTileM * 4);
  const __amdgpu_buffer_rsrc_t tr = make_rsrc(tfrag, tiles_m * 16 * rsteps * 2048);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(lora_b, N * r * 2);
  const uint32_t a_group0 = __builtin_amdgcn_readfirstlane((uint32_t)(2 * tm * ksteps * 8192));
  const uint32_t i_group0 = __builtin_amdgcn_readfirstlane((uint32_t)(2 * tm * ksteps * 1024));
  const uint32_t a_gstride = __builtin_amdgcn_readfirstlane((uint32_t)(ksteps * 8192));
  const uint32_t i_gstride = __builtin_amdgcn_readfirstlane((uint32_t)(ksteps * 1024));
  const uint32_t t_block0 = __builtin_amdgcn_readfirstlane((uint32_t)(tm * 16 * rsteps * 2048));
  const WTileOffsets wo = w_tile_offsets(K, n0);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(&lds[0]);
  constexpr int kWOps = KM == kAligned8 ? 4 * kWChunksPerThread : kWChunksPerThread;
  constexpr int kStepOps = kWOps + 6;

  // Copies of step g (a k-step below ksteps, a LoRA step after) into stage b.
  auto prefetch = [&](int64_t g, int b) {
    const uint32_t st = lds_base + (uint32_t)b * kStageBytes;
    if (RING && g >= ksteps) {
      dma_lora_tile_asm(tr, br, t_block0, rsteps, g - ksteps, N, r, n0, st);
      return;
    }
    dma_a_tile_asm(ar, ir, a_group0, i_group0, a_gstride, i_gstride, g, st);
    if constexpr (KM == kAligned8) dma_w_tile_dword(wr, N, K, n0, g * kTileK, &lds[b * kStageBytes]);
    else dma_w_tile_asm(wr, wo, K, g * kTileK, st, KM == kAligned16);
  };

  const char* b_base0 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(0);
  const char* b_base1 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(1);
  const char* a_base = &lds[0] + kAStageOff + 16 * lane + wm * 8192;
  const char* i_base = &lds[0] + kIStageOff + 16 * lane + wm * 1024;

  // Top of step g in stage b = g % 3: wait until only step g + 1's copies
  // are in flight, barrier (stage b complete for every wave; every wave done
  // with stage (b + 2) % 3), start the copies of step g + 2 (the last step
  // again near the end: a harmless copy into a free stage).
  auto step_top = [&](int64_t g, int b) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kStepOps>();
    barrier_no_fence();
    prefetch(g + 2 < total ? g + 2 : total - 1, (b + 2) % kStages);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One k-step: 8 A fragments and their position fields from LDS, the W
  // fragments (two 16-byte halves per lane, swizzled tile) one column block
  // ahead, 64 structured-sparse MFMAs.  The
  // position fields of row blocks 2j and 2j+1 share a 32-bit word (abid).
  auto kstep = [&](int64_t ks, int b) {
    step_top(ks, b);
    const u32x4 iw = *reinterpret_cast<const u32x4*>(i_base + b * kStageBytes);
    bf16x8 af[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      af[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + b * kStageBytes + rb * 1024));
    const char* s0 = b_base0 + b * kStageBytes;
    const char* s1 = b_base1 + b * kStageBytes;
    u32x4 b0 = *reinterpret_cast<const u32x4*>(s0);
    u32x4 b1 = *reinterpret_cast<const u32x4*>(s1);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x16 bf = __builtin_bit_cast(bf16x16, (u32x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
      if (cb + 1 < kCB) {
        b0 = *reinterpret_cast<const u32x4*>(s0 + (cb + 1) * 2048);
        b1 = *reinterpret_cast<const u32x4*>(s1 + (cb + 1) * 2048);
      }
#pragma unroll
      for (int rb = 0; rb < kRB; rb += 2) {
        acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb], bf, acc[rb][cb], (int)iw[rb / 2], 0, 0);
        acc[rb + 1][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb + 1], bf, acc[rb + 1][cb], (int)iw[rb / 2], 0, 1);
      }
    }
  };

  // One LoRA step: for each half (hi, lo) of alpha T / s, 8 row fragments
  // and 8 B fragments from LDS, 64 dense MFMAs.
  auto lstep = [&](int64_t g, int b) {
    step_top(g, b);
    const char* st = &lds[0] + b * kStageBytes + 16 * lane;
    bf16x8 bfr[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
      bfr[cb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + kAStageOff + (wn * kCB + cb) * 1024));
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      bf16x8 ta[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        ta[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + ((wm * kRB + rb) * 2 + hl) * 1024));
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta[rb], bfr[cb], acc[rb][cb], 0, 0, 0);
    }
  };

  // Prologue: the tile's scales, then steps 0 and 1 (ksteps >= 2 always).
  dma_scale_asm(sr, (uint32_t)(tm * kTileM * 4), lds_base + kScaleOff);
  prefetch(0, 0);
  prefetch(1, 1);
  // One step per iteration, the stage a runtime index: unrolled copies of
  // the step get different accumulator registers from the register
  // allocator, and the copies between them wait on the matrix pipeline.
  int b = 0;
#pragma nounroll
  for (int64_t ks = 0; ks < ksteps; ++ks) {
    kstep(ks, b);
    b = b == kStages - 1 ? 0 : b + 1;
  }
  if constexpr (RING) {
    for (int64_t g = ksteps; g < total; ++g) lstep(g, (int)(g % kStages));
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  barrier_no_fence();                     // every wave is done with the ring

  if constexpr (!RING) {
    // LoRA-up from global memory: (alpha T / s)_hi B^T + (alpha T / s)_lo B^T.
    for (int64_t rs = 0; r > 0 && rs < rsteps; ++rs) {
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

  // Per-token compensation scale on the fp32 accumulators.
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const f32x4 sv = *reinterpret_cast<const f32x4*>(&lds[kScaleOff] + (wm * kWaveM + 16 * rb + 4 * (lane >> 4)) * 4);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rb][cb][i] *= sv[i];
  }

  const int64_t m0 = tm * kTileM + wm * kWaveM;
  if (N % 8 == 0) store_tile_via_lds(acc, lds, y, M, N, m0, n0 + wn * kWaveN);
  else store_acc_bf16(acc, y, M, N, m0, n0 + wn * kWaveN);
}

}  // namespace

hipError_t launch_sparse_gemm(const void* workspace, const uint16_t* w, const uint16_t* lora_b,
                              int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y,
                              hipStream_t stream) {
  const WsLayout L = ws_layout(M, K, r);
  const char* ws = static_cast<const char*>(workspace);
  const u32x4* xv = reinterpret_cast<const u32x4*>(ws + L.off_xv);
  const uint16_t* xi = reinterpret_cast<const uint16_t*>(ws + L.off_xi);
  const float* s = reinterpret_cast<const float*>(ws + L.off_s);
  const u32x4* t = reinterpret_cast<const u32x4*>(ws + L.off_t);
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  const dim3 grid((unsigned)tiles), block(kGemmThreads);
  const int64_t kpairs = L.kp / 128, rsteps = L.rp / 32;
  // The k loop runs over the padded K (a multiple of 128): full-K mode
  // needs K itself to be one.
  const bool ring = r % 8 == 0;
  if (K % 128 == 0 && ring)
    sparse_gemm_kernel<kFullK, true><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y);
  else if (K % 128 == 0)
    sparse_gemm_kernel<kFullK, false><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y);
  else if (K % 8 == 0 && ring)
    sparse_gemm_kernel<kAligned16, true><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y);
  else if (K % 8 == 0)
    sparse_gemm_kernel<kAligned16, false><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y);
  else
    sparse_gemm_kernel<kAligned8, false><<<grid, block, 0, stream>>>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y);
  return hipGetLastError();
}

}  // namespace rtl
