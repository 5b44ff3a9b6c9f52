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
//
// Workgroup: 8 wavefronts, 2 per SIMD, in a 2 (M) x 4 (N) grid of 128 x 64
// tiles (8 x 4 blocks of 16 x 16).  Per k-step a wavefront reads 17 KiB of
// operands from LDS for 32 structured-sparse MFMAs; with one wavefront per
// SIMD (a 128 x 128 tile, 25 KiB for 64 MFMAs) the LDS reads of a single
// wavefront could not keep up with its matrix core.
#include "gemm_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveM = 128, kWaveN = 64;
constexpr int kRB = kWaveM / 16, kCB = kWaveN / 16;          // 8 x 4 blocks per wavefront

// Per k-step LDS stage: the W tile (32 KiB), the workgroup's 256 rows of
// compressed A (16 x 1 KiB fragments) and their position fields (2 x 1 KiB).
// A LoRA step puts the 256 rows of alpha T / s (16 blocks x hi, lo x 1 KiB)
// where W goes and the 256 columns of B (16 x 1 KiB) where A goes.
constexpr int kAStageOff = kTileBytes;
constexpr int kIStageOff = kTileBytes + 16 * 1024;
constexpr int kStageBytes = kTileBytes + 18 * 1024;
constexpr int kStages = 3;                                   // prefetch distance 2
constexpr int kScaleOff = kStages * kStageBytes;             // 256 per-token scales
constexpr int kLdsBytes = kScaleOff + 1024;
static_assert(store_lds_bytes<kRB, kCB>(kWaves) <= kScaleOff, "store staging must not reach the scales");

// Vector-memory operations every step issues per wavefront: 4 for the W
// tile, 2 for the A fragments, 1 for the position fields (a LoRA step pads
// to the same count, so the vmcnt waits are uniform).
constexpr int kWOps = 32 / kWaves;
constexpr int kStepOps = kWOps + 3;

// Copies the compressed A operand of one k-step into an LDS stage: thread
// (wave v, i < 2) moves fragment c = 2 v + i (16-token block c % 8 of group
// c / 8) with one buffer_load_dwordx4 ... lds, and 256 bytes of the position
// fields (part v % 4 of group v / 4's 1 KiB) with one buffer_load_dword ...
// lds.  Same rules as dma_w_tile_asm: no output registers, M0 saved and
// restored, no SCC write.  The instruction offset of a buffer ... lds load
// is added to the LDS address too, so every offset is carried by the scalar
// offset operand.  3 vector-memory operations.
__device__ __forceinline__ void dma_a_tile_asm(__amdgpu_buffer_rsrc_t ar, __amdgpu_buffer_rsrc_t ir,
                                               uint32_t a_group0, uint32_t i_group0, uint32_t a_gstride,
                                               uint32_t i_gstride, int64_t ks, uint32_t lds_stage_addr) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t g = wave >> 2;                       // fragments 2v, 2v+1 lie in group v / 4
  const uint32_t a_so = __builtin_amdgcn_readfirstlane(a_group0 + g * a_gstride + (uint32_t)ks * 8192u +
                                                       (wave & 3u) * 2048u);
  const uint32_t la = __builtin_amdgcn_readfirstlane(lds_stage_addr + kAStageOff + wave * 2048u);
  const uint32_t i_so = __builtin_amdgcn_readfirstlane(i_group0 + g * i_gstride + (uint32_t)ks * 1024u +
                                                       (wave & 3u) * 256u);
  const uint32_t li = __builtin_amdgcn_readfirstlane(lds_stage_addr + kIStageOff + wave * 256u);
  const uint32_t va = 16u * lane, vi = 4u * lane;
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[la0]\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso0] offen lds\n\t"
      "s_mov_b32 m0, %[la1]\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso1] offen lds\n\t"
      "s_mov_b32 m0, %[li0]\n\t"
      "buffer_load_dword %[vi], %[ir], %[iso0] offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [va] "v"(va), [vi] "v"(vi), [ar] "s"(ar), [ir] "s"(ir),
        [aso0] "s"(a_so), [aso1] "s"(a_so + 1024u), [iso0] "s"(i_so),
        [la0] "s"(la), [la1] "s"(la + 1024u), [li0] "s"(li)
      : "memory");
  (void)saved;
}

// Copies the operands of LoRA step rs into an LDS stage: thread (wave v,
// i < 4) moves 1 KiB of alpha T / s (16-token block 2 v + i / 2, half i % 2)
// and thread (v, i < 2) 1 KiB of B (columns n0 + 16 (2 v + i) + [0, 16),
// ranks 32 rs + 8 (l / 16) + [0, 8)).  B rows past N and rank chunks past r
// carry their whole offset in the VGPR operand and read as zeros.  The
// last B copy is issued twice, so that a LoRA step issues as many
// vector-memory operations (7) as a k-step.
__device__ __forceinline__ void dma_lora_tile_asm(__amdgpu_buffer_rsrc_t tr, __amdgpu_buffer_rsrc_t br,
                                                  uint32_t t_block0, int64_t rsteps, int64_t rs,
                                                  int64_t N, int64_t r, int64_t n0, uint32_t lds_stage_addr) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t blk = __builtin_amdgcn_readfirstlane((uint32_t)(rsteps * 2048));
  const uint32_t t_so = __builtin_amdgcn_readfirstlane(t_block0 + 2u * wave * blk + (uint32_t)rs * 2048u);
  const uint32_t lt = __builtin_amdgcn_readfirstlane(lds_stage_addr + wave * 4096u);
  const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_stage_addr + kAStageOff + wave * 2048u);
  const uint32_t vt = 16u * lane;
  const int64_t j = 32 * rs + 8 * (lane >> 4);
  uint32_t vb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 16 * (2 * (int64_t)wave + i) + (lane & 15);
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
      "s_mov_b32 m0, %[lb0]\n\t"
      "buffer_load_dwordx4 %[vb0], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb1]\n\t"
      "buffer_load_dwordx4 %[vb1], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[lb1]\n\t"
      "buffer_load_dwordx4 %[vb1], %[br], 0 offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [vt] "v"(vt), [vb0] "v"(vb[0]), [vb1] "v"(vb[1]), [tr] "s"(tr), [br] "s"(br),
        [ts0] "s"(t_so), [ts1] "s"(t_so + 1024u), [ts2] "s"(t_so + blk), [ts3] "s"(t_so + blk + 1024u),
        [lt0] "s"(lt), [lt1] "s"(lt + 1024u), [lt2] "s"(lt + 2048u), [lt3] "s"(lt + 3072u),
        [lb0] "s"(lb), [lb1] "s"(lb + 1024u)
      : "memory");
  (void)saved;
}

// Copies the workgroup's 256 per-token scales into LDS: wavefronts 0-3 move
// 64 each with one dword DMA.  (The other wavefronts issue nothing; the
// vmcnt waits after it only bound later operations, so they hold for both.)
__device__ __forceinline__ void dma_scale_asm(__amdgpu_buffer_rsrc_t sr, uint32_t row0_bytes,
                                              uint32_t lds_scale_addr) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4) return;
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
__global__ void __launch_bounds__(kThreads, 1)
sparse_gemm_kernel(const u32x4* __restrict__ xv, const uint16_t* __restrict__ xi,
                   const float* __restrict__ s, const u32x4* __restrict__ tfrag,
                   const uint16_t* __restrict__ w, const uint16_t* __restrict__ lora_b,
                   int64_t M, int64_t N, int64_t K, int64_t r, int64_t kpairs,
                   int64_t rsteps, uint16_t* __restrict__ y) {
  static_assert(!RING || KM != kAligned8, "the ring's uniform waits need 7 operations per step");
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
  const int wm = wave >> 2, wn = wave & 3;
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
  const WTileOffsets wo = w_tile_offsets<kWaves>(K, n0);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(&lds[0]);

  // Copies of step g (a k-step below ksteps, a LoRA step after) into stage b.
  auto prefetch = [&](int64_t g, int b) {
    const uint32_t st = lds_base + (uint32_t)b * kStageBytes;
    if (RING && g >= ksteps) {
      dma_lora_tile_asm(tr, br, t_block0, rsteps, g - ksteps, N, r, n0, st);
      return;
    }
    dma_a_tile_asm(ar, ir, a_group0, i_group0, a_gstride, i_gstride, g, st);
    if constexpr (KM == kAligned8) dma_w_tile_dword<kWaves>(wr, N, K, n0, g * kTileK, &lds[b * kStageBytes]);
    else dma_w_tile_asm<kWaves>(wr, wo, K, g * kTileK, st, KM == kAligned16);
  };
  constexpr int kOps = KM == kAligned8 ? 128 / kWaves + 3 : kStepOps;

  const char* b_base0 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(0);
  const char* b_base1 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(1);
  const char* a_base = &lds[0] + kAStageOff + 16 * lane + wm * 8192;
  const char* i_base = &lds[0] + kIStageOff + 16 * lane + wm * 1024;

  // Two barriers per step g (stage b = g % 3):
  //  * at the top: every wave is done with step g - 1, so its stage
  //    (b + 2) % 3 is free and the copies of step g + 2 start there (near
  //    the end, the last step again: a harmless copy into a free stage);
  //  * before the last column block: each wave has waited for its copies of
  //    step g + 1 (only step g + 2's may be in flight), so after the barrier
  //    stage (b + 1) % 3 is complete.  The last column block's MFMAs then
  //    overlap the LDS reads of step g + 1's first operands, and the next
  //    step starts its MFMAs without a load bubble.
  // A copy issued at the top of step g - 1 thus has until late in step g.
  auto barrier_top = [&](int64_t g, int b) {
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();
    prefetch(g + 2 < total ? g + 2 : total - 1, (b + 2) % kStages);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto barrier_mid = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kOps>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Operands a k-step starts with: the position fields, the 8 A fragments
  // and the first column block of W, read from stage b.
  u32x4 iw, bq0, bq1;
  bf16x8 af[kRB];
  auto load_first = [&](int b) {
    iw = *reinterpret_cast<const u32x4*>(i_base + b * kStageBytes);
    bq0 = *reinterpret_cast<const u32x4*>(b_base0 + b * kStageBytes);
    bq1 = *reinterpret_cast<const u32x4*>(b_base1 + b * kStageBytes);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      af[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + b * kStageBytes + rb * 1024));
  };

  // One k-step: 32 structured-sparse MFMAs, the W fragments (two 16-byte
  // halves per lane, swizzled tile) read one column block ahead.  The
  // position fields of row blocks 2j and 2j+1 share a 32-bit word (abid).
  auto kstep = [&](int64_t ks, int b) {
    barrier_top(ks, b);
    const char* s0 = b_base0 + b * kStageBytes;
    const char* s1 = b_base1 + b * kStageBytes;
    const int bn = b == kStages - 1 ? 0 : b + 1;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x16 bf = __builtin_bit_cast(bf16x16, (u32x8){bq0[0], bq0[1], bq0[2], bq0[3], bq1[0], bq1[1], bq1[2], bq1[3]});
      if (cb + 1 < kCB) {
        bq0 = *reinterpret_cast<const u32x4*>(s0 + (cb + 1) * 2048);
        bq1 = *reinterpret_cast<const u32x4*>(s1 + (cb + 1) * 2048);
#pragma unroll
        for (int rb = 0; rb < kRB; rb += 2) {
          acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb], bf, acc[rb][cb], (int)iw[rb / 2], 0, 0);
          acc[rb + 1][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb + 1], bf, acc[rb + 1][cb], (int)iw[rb / 2], 0, 1);
        }
      } else {
        barrier_mid();
        const u32x4 iw_cur = iw;
        iw = *reinterpret_cast<const u32x4*>(i_base + bn * kStageBytes);
        bq0 = *reinterpret_cast<const u32x4*>(b_base0 + bn * kStageBytes);
        bq1 = *reinterpret_cast<const u32x4*>(b_base1 + bn * kStageBytes);
#pragma unroll
        for (int rb = 0; rb < kRB; rb += 2) {
          acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb], bf, acc[rb][cb], (int)iw_cur[rb / 2], 0, 0);
          acc[rb + 1][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb + 1], bf, acc[rb + 1][cb], (int)iw_cur[rb / 2], 0, 1);
          af[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + bn * kStageBytes + rb * 1024));
          af[rb + 1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + bn * kStageBytes + (rb + 1) * 1024));
        }
        // Interleave: the 3 reads above first, then one MFMA and one read
        // (the A fragment the MFMA has just consumed) at a time.
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // One LoRA step: for each half (hi, lo) of alpha T / s, 8 row fragments
  // and 4 B fragments from LDS, 32 dense MFMAs; then the wait and barrier
  // that make the next step's stage complete.
  auto lstep = [&](int64_t g, int b) {
    barrier_top(g, b);
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
    barrier_mid();
  };

  // Prologue: the tile's scales, then steps 0 and 1 (ksteps >= 2 always);
  // wait for step 0 and read its first operands.
  dma_scale_asm(sr, (uint32_t)(tm * kTileM * 4), lds_base + kScaleOff);
  prefetch(0, 0);
  prefetch(1, 1);
  barrier_mid();
  load_first(0);
  // One step per iteration, the stage a runtime index: unrolled copies of
  // the step get different accumulator registers from the register
  // allocator, and the copies between them wait on the matrix pipeline.
  // (After the last k-step the operands read for "the next step" are
  // unused.)
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
  if (N % 8 == 0) store_tile_via_lds<kRB, kCB>(acc, lds, y, M, N, m0, n0 + wn * kWaveN);
  else store_acc_bf16<kRB, kCB>(acc, y, M, N, m0, n0 + wn * kWaveN);
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
  const dim3 grid((unsigned)tiles), block(kThreads);
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
