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
constexpr int kScaleOff = kStages * kStageBytes;             // 2 x 256 per-token scales
constexpr int kLdsBytes = kScaleOff + 2048;
static_assert(kWaves * 32 * store_pitch<kCB>() <= kStageBytes, "store staging (2 row blocks) fits one stage");

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

// Persistent: the grid holds at most one workgroup per CU, and workgroup w
// computes tiles w, w + G, w + 2G, ... (G = grid size; these run on w's XCD,
// see tile_coords_of).  All steps of all its tiles form one pipeline: the
// copies of the next tile's first two steps are in flight while the current
// tile's epilogue scales and stores it through the one free stage.
//
// RING: the LoRA-up runs as extra steps of the LDS ring (r % 8 == 0 and
// 16-byte W rows).  Otherwise it runs in the epilogue from global memory
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
  const int64_t ntiles = tiles_m * tiles_n;
  const int64_t G = gridDim.x;
  const int64_t my_tiles = (ntiles - (int64_t)blockIdx.x + G - 1) / G;   // >= 1: grid <= tiles
  const int64_t ksteps = 2 * kpairs;
  const int64_t lsteps = RING && r > 0 ? rsteps : 0;
  const int64_t spt = ksteps + lsteps;                  // steps per tile

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
  const uint32_t a_gstride = __builtin_amdgcn_readfirstlane((uint32_t)(ksteps * 8192));
  const uint32_t i_gstride = __builtin_amdgcn_readfirstlane((uint32_t)(ksteps * 1024));
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(&lds[0]);
  constexpr int kOps = KM == kAligned8 ? 128 / kWaves + 3 : kStepOps;

  // Prefetch cursor: the step the next prefetch copies (tile ordinal, step
  // within the tile, and that tile's copy offsets).  After the last step of
  // the last tile it stays there: the extra copies are harmless copies into
  // free stages.
  int64_t pc_i = 0, pc_loc = 0, pc_n0 = 0;
  uint32_t pc_ag0 = 0, pc_ig0 = 0, pc_tb0 = 0;
  WTileOffsets pc_wo;
  auto cursor_tile = [&](int64_t i) {
    int64_t tm, tn;
    tile_coords_of((int64_t)blockIdx.x + i * G, tiles_m, tiles_n, tm, tn);
    pc_n0 = tn * kTileN;
    pc_ag0 = __builtin_amdgcn_readfirstlane((uint32_t)(2 * tm * ksteps * 8192));
    pc_ig0 = __builtin_amdgcn_readfirstlane((uint32_t)(2 * tm * ksteps * 1024));
    pc_tb0 = __builtin_amdgcn_readfirstlane((uint32_t)(tm * 16 * rsteps * 2048));
    pc_wo = w_tile_offsets<kWaves>(K, pc_n0);
  };
  cursor_tile(0);
  auto prefetch = [&](int b) {
    const uint32_t st = lds_base + (uint32_t)b * kStageBytes;
    if (RING && pc_loc >= ksteps) {
      dma_lora_tile_asm(tr, br, pc_tb0, rsteps, pc_loc - ksteps, N, r, pc_n0, st);
    } else {
      dma_a_tile_asm(ar, ir, pc_ag0, pc_ig0, a_gstride, i_gstride, pc_loc, st);
      if constexpr (KM == kAligned8) dma_w_tile_dword<kWaves>(wr, N, K, pc_n0, pc_loc * kTileK, &lds[b * kStageBytes]);
      else dma_w_tile_asm<kWaves>(wr, pc_wo, K, pc_loc * kTileK, st, KM == kAligned16);
    }
    if (pc_loc + 1 < spt) {
      ++pc_loc;
    } else if (pc_i + 1 < my_tiles) {
      ++pc_i;
      pc_loc = 0;
      cursor_tile(pc_i);
    }
  };
  // Per-token scales of tile i into LDS buffer i % 2.
  auto copy_scales = [&](int64_t i) {
    int64_t tm, tn;
    tile_coords_of((int64_t)blockIdx.x + i * G, tiles_m, tiles_n, tm, tn);
    dma_scale_asm(sr, (uint32_t)(tm * kTileM * 4), lds_base + kScaleOff + (uint32_t)(i & 1) * 1024u);
  };

  const char* b_base0 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(0);
  const char* b_base1 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(1);
  const char* a_base = &lds[0] + kAStageOff + 16 * lane + wm * 8192;
  const char* i_base = &lds[0] + kIStageOff + 16 * lane + wm * 1024;

  // Two barriers per step (stage b):
  //  * at the top: every wave is done with the previous step, so its stage
  //    (b + 2) % 3 is free and the copies two steps ahead start there (with
  //    the next tile's scales on a tile's first step);
  //  * before the last column block: each wave has waited for its copies of
  //    the next step (only those two steps ahead may be in flight), so after
  //    the barrier stage (b + 1) % 3 is complete.  The last column block's
  //    MFMAs then overlap the LDS reads of the next step's first operands,
  //    and the next step starts its MFMAs without a load bubble.
  // A copy issued at the top of one step thus has until late in the next.
  auto barrier_top = [&](int b, int64_t scales_for) {
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();
    prefetch((b + 2) % kStages);
    if (scales_for >= 0) copy_scales(scales_for);
    __builtin_amdgcn_sched_barrier(0);
  };
  // after_stores: the previous tile's output stores were issued after the
  // awaited copies and may still be in flight (vmcnt counts them too).
  constexpr int kStoreOps = store_passes_ops<kRB, kCB, 2>();
  static_assert(kOps + kStoreOps < 64, "vmcnt field is 6 bits");
  auto barrier_mid = [&](bool after_stores = false) {
    __builtin_amdgcn_sched_barrier(0);
    if (after_stores) wait_vm<kOps + kStoreOps>();
    else wait_vm<kOps>();
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

  f32x4 acc[kRB][kCB];

  // One k-step: 32 structured-sparse MFMAs, the W fragments (two 16-byte
  // halves per lane, swizzled tile) read one column block ahead.  The
  // position fields of row blocks 2j and 2j+1 share a 32-bit word (abid).
  auto kstep = [&](int b, int64_t scales_for, bool after_stores) {
    barrier_top(b, scales_for);
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
        barrier_mid(after_stores);
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
  auto lstep = [&](int b) {
    barrier_top(b, -1);
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

  // Prologue: the first tile's scales, then its steps 0 and 1 (ksteps >= 2
  // always); wait for step 0 and read its first operands.
  copy_scales(0);
  prefetch(0);
  prefetch(1);
  barrier_mid();
  load_first(0);

  int b = 0;
  for (int64_t i = 0; i < my_tiles; ++i) {
    int64_t tm, tn;
    tile_coords_of((int64_t)blockIdx.x + i * G, tiles_m, tiles_n, tm, tn);
    const int64_t n0 = tn * kTileN;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) acc[rb][cb] = (f32x4){0, 0, 0, 0};

    // One step per iteration, the stage a runtime index: unrolled copies of
    // the step get different accumulator registers from the register
    // allocator, and the copies between them wait on the matrix pipeline.
    // The first step also copies the next tile's scales.
    kstep(b, i + 1 < my_tiles ? i + 1 : -1, i > 0 && N % 8 == 0);
    b = b == kStages - 1 ? 0 : b + 1;
#pragma nounroll
    for (int64_t ks = 1; ks < ksteps; ++ks) {
      kstep(b, -1, false);
      b = b == kStages - 1 ? 0 : b + 1;
    }
    if constexpr (RING) {
      for (int64_t g = 0; g < lsteps; ++g) {
        lstep(b);
        b = b == kStages - 1 ? 0 : b + 1;
      }
    }
    // Epilogue.  Every wave has consumed the last step's stage (the barrier
    // below), the next stage is complete and the one after is in flight.
    const int b_last = b == 0 ? kStages - 1 : b - 1;
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();

    if constexpr (!RING) {
      // LoRA-up from global memory: (alpha T / s)_hi B^T + (alpha T / s)_lo B^T.
      const int64_t mb0 = (tm * kTileM + wm * kWaveM) / 16;
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

    // Per-token compensation scale on the fp32 accumulators.  (Tile i's
    // scales were copied two tiles' worth of steps ago, or in the prologue.)
    const char* sbuf = &lds[kScaleOff] + (i & 1) * 1024;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const f32x4 sv = *reinterpret_cast<const f32x4*>(sbuf + (wm * kWaveM + 16 * rb + 4 * (lane >> 4)) * 4);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) acc[rb][cb][i4] *= sv[i4];
    }

    const int64_t m0 = tm * kTileM + wm * kWaveM;
    if (N % 8 == 0) {
      char* region = &lds[0] + b_last * kStageBytes + wave * (32 * store_pitch<kCB>());
      store_tile_via_lds_passes<kRB, kCB, 2>(acc, region, y, M, N, m0, n0 + wn * kWaveN);
    } else {
      store_acc_bf16<kRB, kCB>(acc, y, M, N, m0, n0 + wn * kWaveN);
    }
    // The next tile starts from stage b, complete since the last step's
    // second barrier.
    if (i + 1 < my_tiles) load_first(b);
  }
  // Drain the remaining (redundant) copies before the workgroup's LDS is
  // released.
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
}

}  // namespace

hipError_t launch_sparse_gemm(const void* workspace, const uint16_t* w, const uint16_t* lora_b,
                              int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y,
                              int compute_units, hipStream_t stream) {
  const WsLayout L = ws_layout(M, K, r);
  const char* ws = static_cast<const char*>(workspace);
  const u32x4* xv = reinterpret_cast<const u32x4*>(ws + L.off_xv);
  const uint16_t* xi = reinterpret_cast<const uint16_t*>(ws + L.off_xi);
  const float* s = reinterpret_cast<const float*>(ws + L.off_s);
  const u32x4* t = reinterpret_cast<const u32x4*>(ws + L.off_t);
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  // One persistent workgroup per CU (the LDS allows one), at most one per tile.
  const int64_t cus = compute_units > 0 ? compute_units : 1;
  const dim3 grid((unsigned)(tiles < cus ? tiles : cus)), block(kThreads);
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
