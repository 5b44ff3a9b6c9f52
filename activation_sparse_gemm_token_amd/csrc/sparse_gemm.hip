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
constexpr int kWaveM = 128;
constexpr int kRB = kWaveM / 16;                              // 8 row blocks per wavefront
constexpr int kStages = 3;                                   // prefetch distance 2

// Tile of 256 rows x 64 CB columns (CB = 4: 256, the default; CB = 3: 192,
// for widths whose 256-column tiles would leave CUs idle): 8 wavefronts in
// a 2 (M) x 4 (N) grid of 128 x 16 CB tiles (8 x CB blocks of 16 x 16).
//
// Per k-step LDS stage: the W tile (CB x 8 KiB), the workgroup's 256 rows of
// compressed A (16 x 1 KiB fragments) and their position fields (2 x 1 KiB).
// A LoRA step puts the 256 rows of alpha T / s (16 blocks x hi, lo x 1 KiB)
// at the start of the stage and the tile's columns of B (4 CB x 1 KiB) after
// them.  Two 1 KiB buffers of per-token scales follow the stages.
template <int CB>
struct Tile {
  static constexpr int kCB = CB;
  static constexpr int kWaveN = 16 * CB;
  static constexpr int kTileNc = 4 * kWaveN;                 // 256 or 192 columns
  static constexpr int kWBytes = kTileNc * 128;
  static constexpr int kAStageOff = kWBytes;
  static constexpr int kIStageOff = kWBytes + 16 * 1024;
  static constexpr int kLoraBOff = 32 * 1024;
  static constexpr int kKStepBytes = kWBytes + 18 * 1024;
  static constexpr int kLoraBytes = kLoraBOff + 4 * CB * 1024;
  static constexpr int kStageBytes = kKStepBytes > kLoraBytes ? kKStepBytes : kLoraBytes;
  static constexpr int kScaleOff = kStages * kStageBytes;
  static constexpr int kProbeOff = kScaleOff + 2048;          // 8 x 256 B, L2 prefetch probes
  static constexpr int kLdsBytes = kProbeOff + 2048;
  // Vector-memory operations every step issues per wavefront: CB for the W
  // tile, 2 for the A fragments, 1 for the position fields (a LoRA step
  // pads to the same count, so the vmcnt waits are uniform).
  static constexpr int kWOps = CB;
  static constexpr int kStepOps = CB + 3;
  static_assert(kWaves * 32 * store_pitch<CB>() <= kStageBytes, "store staging (2 row blocks) fits one stage");
  static_assert(kWaves * 16 * store_pitch<CB>() <= kStageBytes - kAStageOff, "1 row block fits the A region");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// Copies of one k-step, issued by every wavefront into the stage at LDS
// address `stage`, CB + 3 vector-memory operations:
//  * its 8 CB rows of the W tile: CB buffer_load_dwordx4 ... lds of 8 rows x
//    128 bytes (whole lines, swizzled as described for the W tile);
//    per-lane row offsets w[i] (VGPR), channel offset w_so (SGPR);
//  * A fragments 2 v and 2 v + 1 (16-token block 2 v % 8 + [0, 2) of group
//    v / 4): one 1 KiB buffer_load_dwordx4 ... lds each, source a_so; the
//    second uses the instruction offset 1024, which moves the global and
//    the LDS address alike;
//  * 256 bytes of the position fields (part v % 4 of group v / 4) with one
//    buffer_load_dword ... lds, source i_so.
// The block builds every LDS destination in M0 from `stage` and the
// wavefront's constant offsets (lw, la, li), saves and restores M0, and
// keeps one wait state between each M0 write and the copy that reads it.
// It clobbers SCC.  s_nop 4 covers a VALU write of an SGPR operand right
// before the block.  Nothing here is visible to the compiler as a load: the
// caller waits with explicit vmcnt counts.
template <int CB>
__device__ __forceinline__ void dma_kstep_asm(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t ar,
                                              __amdgpu_buffer_rsrc_t ir, const uint32_t (&w)[CB],
                                              uint32_t w_so, uint32_t a_so, uint32_t i_so, uint32_t va,
                                              uint32_t vi, uint32_t stage, uint32_t lw, uint32_t la,
                                              uint32_t li) {
  static_assert(CB == 3 || CB == 4, "192- or 256-column tiles");
  uint32_t saved;
  if constexpr (CB == 4) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_add_u32 m0, %[st], %[lw]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w0], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w1], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w2], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w3], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, %[st], %[la]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[va], %[ar], %[aso] offen lds\n\t"
        "buffer_load_dwordx4 %[va], %[ar], %[aso] offen offset:1024 lds\n\t"
        "s_add_u32 m0, %[st], %[li]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %[vi], %[ir], %[iso] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [va] "v"(va), [vi] "v"(vi),
          [wr] "s"(wr), [ar] "s"(ar), [ir] "s"(ir), [wso] "s"(w_so), [aso] "s"(a_so), [iso] "s"(i_so),
          [st] "s"(stage), [lw] "s"(lw), [la] "s"(la), [li] "s"(li)
        : "memory", "scc");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_add_u32 m0, %[st], %[lw]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w0], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w1], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w2], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, %[st], %[la]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[va], %[ar], %[aso] offen lds\n\t"
        "buffer_load_dwordx4 %[va], %[ar], %[aso] offen offset:1024 lds\n\t"
        "s_add_u32 m0, %[st], %[li]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %[vi], %[ir], %[iso] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [va] "v"(va), [vi] "v"(vi),
          [wr] "s"(wr), [ar] "s"(ar), [ir] "s"(ir), [wso] "s"(w_so), [aso] "s"(a_so), [iso] "s"(i_so),
          [st] "s"(stage), [lw] "s"(lw), [la] "s"(la), [li] "s"(li)
        : "memory", "scc");
  }
  (void)saved;
}

// The A fragments and position fields of dma_kstep_asm alone (3
// operations), for rows of W that are only 8-byte aligned (K % 8 == 4),
// whose tile goes through the compiler-visible dword copy.
__device__ __forceinline__ void dma_a_tile_asm(__amdgpu_buffer_rsrc_t ar, __amdgpu_buffer_rsrc_t ir,
                                               uint32_t a_so, uint32_t i_so, uint32_t va, uint32_t vi,
                                               uint32_t stage, uint32_t la, uint32_t li) {
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_add_u32 m0, %[st], %[la]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso] offen lds\n\t"
      "buffer_load_dwordx4 %[va], %[ar], %[aso] offen offset:1024 lds\n\t"
      "s_add_u32 m0, %[st], %[li]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %[vi], %[ir], %[iso] offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [va] "v"(va), [vi] "v"(vi), [ar] "s"(ar), [ir] "s"(ir), [aso] "s"(a_so), [iso] "s"(i_so),
        [st] "s"(stage), [la] "s"(la), [li] "s"(li)
      : "memory", "scc");
  (void)saved;
}

// The W tile of dma_kstep_asm alone (CB operations).
template <int CB>
__device__ __forceinline__ void dma_w_tile_part_asm(__amdgpu_buffer_rsrc_t wr, const uint32_t (&w)[CB],
                                                    uint32_t w_so, uint32_t stage, uint32_t lw) {
  uint32_t saved;
  if constexpr (CB == 4) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_add_u32 m0, %[st], %[lw]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w0], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w1], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w2], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w3], %[wr], %[wso] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [wr] "s"(wr), [wso] "s"(w_so),
          [st] "s"(stage), [lw] "s"(lw)
        : "memory", "scc");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_add_u32 m0, %[st], %[lw]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w0], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w1], %[wr], %[wso] offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[w2], %[wr], %[wso] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [wr] "s"(wr), [wso] "s"(w_so),
          [st] "s"(stage), [lw] "s"(lw)
        : "memory", "scc");
  }
  (void)saved;
}

// Copies the operands of LoRA step rs into an LDS stage: thread (wave v,
// i < 4) moves 1 KiB of alpha T / s (16-token block 2 v + i / 2, half i % 2)
// to the start of the stage, and thread (v, i < 2) 1 KiB of B, fragments v
// and v + 8 of the tile's 4 CB (columns n0 + 16 f + [0, 16), ranks
// 32 rs + 8 (l / 16) + [0, 8)) to kLoraBOff + 1 KiB f; a fragment index past
// the tile repeats fragment v.  B rows past N and rank chunks past r carry
// their whole offset in the VGPR operand and read as zeros.  The last copy
// is repeated until the step has issued as many vector-memory operations
// (OPS) as a k-step.
template <int CB, int OPS>
__device__ __forceinline__ void dma_lora_tile_asm(__amdgpu_buffer_rsrc_t tr, __amdgpu_buffer_rsrc_t br,
                                                  uint32_t t_block0, int64_t rsteps, int64_t rs,
                                                  int64_t N, int64_t r, int64_t n0, uint32_t lds_stage_addr) {
  static_assert(OPS == 6 || OPS == 7, "4 + 2 copies, padded to a k-step's count");
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t blk = __builtin_amdgcn_readfirstlane((uint32_t)(rsteps * 2048));
  const uint32_t t_so = __builtin_amdgcn_readfirstlane(t_block0 + 2u * wave * blk + (uint32_t)rs * 2048u);
  const uint32_t lt = __builtin_amdgcn_readfirstlane(lds_stage_addr + wave * 4096u);
  const uint32_t f1 = wave + 8u < 4u * CB ? wave + 8u : wave;
  const uint32_t lb0 = __builtin_amdgcn_readfirstlane(lds_stage_addr + Tile<CB>::kLoraBOff + wave * 1024u);
  const uint32_t lb1 = __builtin_amdgcn_readfirstlane(lds_stage_addr + Tile<CB>::kLoraBOff + f1 * 1024u);
  const uint32_t vt = 16u * lane;
  const int64_t j = 32 * rs + 8 * (lane >> 4);
  uint32_t vb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 16 * (int64_t)(i == 0 ? wave : f1) + (lane & 15);
    vb[i] = (n < N && j + 8 <= r) ? (uint32_t)((n * r + j) * 2) : kOobOffset;
  }
  uint32_t saved;
  if constexpr (OPS == 7) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[lt0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts0] offen lds\n\t"
        "s_mov_b32 m0, %[lt1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts1] offen lds\n\t"
        "s_mov_b32 m0, %[lt2]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts2] offen lds\n\t"
        "s_mov_b32 m0, %[lt3]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts3] offen lds\n\t"
        "s_mov_b32 m0, %[lb0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vb0], %[br], 0 offen lds\n\t"
        "s_mov_b32 m0, %[lb1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vb1], %[br], 0 offen lds\n\t"
        "buffer_load_dwordx4 %[vb1], %[br], 0 offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [vt] "v"(vt), [vb0] "v"(vb[0]), [vb1] "v"(vb[1]), [tr] "s"(tr), [br] "s"(br),
          [ts0] "s"(t_so), [ts1] "s"(t_so + 1024u), [ts2] "s"(t_so + blk), [ts3] "s"(t_so + blk + 1024u),
          [lt0] "s"(lt), [lt1] "s"(lt + 1024u), [lt2] "s"(lt + 2048u), [lt3] "s"(lt + 3072u),
          [lb0] "s"(lb0), [lb1] "s"(lb1)
        : "memory");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[lt0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts0] offen lds\n\t"
        "s_mov_b32 m0, %[lt1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts1] offen lds\n\t"
        "s_mov_b32 m0, %[lt2]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts2] offen lds\n\t"
        "s_mov_b32 m0, %[lt3]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vt], %[tr], %[ts3] offen lds\n\t"
        "s_mov_b32 m0, %[lb0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vb0], %[br], 0 offen lds\n\t"
        "s_mov_b32 m0, %[lb1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[vb1], %[br], 0 offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [vt] "v"(vt), [vb0] "v"(vb[0]), [vb1] "v"(vb[1]), [tr] "s"(tr), [br] "s"(br),
          [ts0] "s"(t_so), [ts1] "s"(t_so + 1024u), [ts2] "s"(t_so + blk), [ts3] "s"(t_so + blk + 1024u),
          [lt0] "s"(lt), [lt1] "s"(lt + 1024u), [lt2] "s"(lt + 2048u), [lt3] "s"(lt + 3072u),
          [lb0] "s"(lb0), [lb1] "s"(lb1)
        : "memory");
  }
  (void)saved;
}

// L2 prefetch probe: one dword per lane by DMA into a throwaway LDS area
// (no register is written, so nothing waits for it); lanes given
// kOobOffset touch no memory.  One vector-memory operation.
__device__ __forceinline__ void l2_probe_asm(__amdgpu_buffer_rsrc_t wr, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[l]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %[v], %[rs], 0 offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [v] "v"(voff), [rs] "s"(wr), [l] "s"(lds_addr)
      : "memory");
  (void)saved;
}

// Copies the workgroup's 256 per-token scales into LDS: wavefronts 0-3 move
// 64 each with one dword DMA.  (The other wavefronts issue nothing; the
// vmcnt waits after it only bound later operations, so they hold for both.)
__device__ __forceinline__ void dma_scale_asm(__amdgpu_buffer_rsrc_t sr, uint32_t row0_bytes,
                                              uint32_t lds_scale_addr, uint32_t v /* 4 lane */) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4) return;
  const uint32_t so = __builtin_amdgcn_readfirstlane(row0_bytes + 256u * wave);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(lds_scale_addr + 256u * wave);
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[ls]\n\t"
      "s_nop 0\n\t"
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
//
// PFW (weights expected cold, only with RING): every k-step one wavefront
// in turn probes 32 rows of the W slice kPfDist steps past the one being
// copied, one dword per 128-byte line, so that the line is on its way from
// HBM into L2 when its copy is issued; the 8 workgroups of an XCD that
// share a W slice (an 8 x 4 block of tiles, tile_coords_of) probe its 256
// rows between them, by tile row.  A tile's first kPfDist steps are not
// probed.  The probes' completion is never awaited: the issuing
// wavefront's vmcnt waits then also cover them, which only makes those
// waits stricter.
template <int KM, bool RING, int CB, bool PFW>
__global__ void __launch_bounds__(kThreads, 1)
sparse_gemm_kernel(const u32x4* __restrict__ xv, const uint16_t* __restrict__ xi,
                   const float* __restrict__ s, const u32x4* __restrict__ tfrag,
                   const uint16_t* __restrict__ w, const uint16_t* __restrict__ lora_b,
                   int64_t M, int64_t N, int64_t K, int64_t r, int64_t kpairs,
                   int64_t rsteps, uint16_t* __restrict__ y) {
  static_assert(!RING || KM != kAligned8, "the ring's uniform waits need CB + 3 operations per step");
  static_assert(RING || !PFW, "W probes come with the ring");
  static_assert(CB == 4 || KM != kAligned8, "the dword tile copy moves 256 rows");
  using T = Tile<CB>;
  constexpr int kCB = CB, kWaveN = T::kWaveN, kTileN = T::kTileNc;
  constexpr int kAStageOff = T::kAStageOff, kIStageOff = T::kIStageOff, kStageBytes = T::kStageBytes;
  constexpr int kScaleOff = T::kScaleOff;
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (N + kTileN - 1) / kTileN;
  const int64_t ntiles = tiles_m * tiles_n;
  const int G = gridDim.x;
  const int my_tiles = (int)((ntiles - (int64_t)blockIdx.x + G - 1) / G);   // >= 1: grid <= tiles
  const int ksteps = 2 * (int)kpairs;
  const int lsteps = RING && r > 0 ? (int)rsteps : 0;
  const int spt = ksteps + lsteps;                      // steps per tile

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
  // Byte offsets below are 32-bit: the host keeps every tensor and
  // workspace region (with 256 rows of padding) under 2 GiB.
  const uint32_t a_gstride = __builtin_amdgcn_readfirstlane((uint32_t)(ksteps * 8192));
  const uint32_t i_gstride = __builtin_amdgcn_readfirstlane((uint32_t)(ksteps * 1024));
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(&lds[0]);
  constexpr int kOps = KM == kAligned8 ? 128 / kWaves + 3 : T::kStepOps;

  // The wavefront's share of a k-step copy: LDS offsets inside a stage and
  // per-lane source offsets (see dma_kstep_asm).
  const uint32_t lw = __builtin_amdgcn_readfirstlane(1024u * kCB * (uint32_t)wave);
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)kAStageOff + 2048u * (uint32_t)wave);
  const uint32_t li = __builtin_amdgcn_readfirstlane((uint32_t)kIStageOff + 256u * (uint32_t)wave);
  const uint32_t row8 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * K));
  const uint32_t k_lane = 8u * (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t va = 16u * (uint32_t)lane, vi = 4u * (uint32_t)lane;
  const uint32_t a_wave = __builtin_amdgcn_readfirstlane((uint32_t)(wave >> 2) * a_gstride + (uint32_t)(wave & 3) * 2048u);
  const uint32_t i_wave = __builtin_amdgcn_readfirstlane((uint32_t)(wave >> 2) * i_gstride + (uint32_t)(wave & 3) * 256u);

  // Prefetch cursor: the step the next prefetch copies (tile ordinal and
  // step within the tile) and, for its k-steps, the copy offsets, advanced
  // by a constant per step.  After the last step of the last tile it stays
  // there: the extra copies are harmless repeats into free stages.
  int pc_i = 0, pc_loc = 0;
  int64_t pc_n0 = 0;
  uint32_t pf_r0 = 0;   // PFW: the first of the 32 W rows this workgroup probes in the cursor's tile
  uint32_t pc_tb0 = 0, pc_wso = 0, pc_aso = 0, pc_iso = 0, pc_wv = 0;
  auto cursor_tile = [&](int i) {
    int64_t tm, tn;
    tile_coords_of((int64_t)blockIdx.x + (int64_t)i * G, tiles_m, tiles_n, tm, tn);
    pc_n0 = tn * kTileN;
    if constexpr (PFW) pf_r0 = __builtin_amdgcn_readfirstlane((uint32_t)(pc_n0 + 32 * (tm & 7)));
    pc_aso = __builtin_amdgcn_readfirstlane((uint32_t)(2 * tm * ksteps * 8192) + a_wave);
    pc_iso = __builtin_amdgcn_readfirstlane((uint32_t)(2 * tm * ksteps * 1024) + i_wave);
    pc_tb0 = __builtin_amdgcn_readfirstlane((uint32_t)(tm * 16 * rsteps * 2048));
    pc_wso = 0;
    pc_wv = (uint32_t)(((pc_n0 + 8 * kCB * wave + (lane >> 3)) * K) * 2) + 2u * k_lane;
  };
  cursor_tile(0);
  // part: 0 the whole step; 1 its W tile only (a k-step of the ring in the
  // 16-byte copy modes; the cursor stays); 2 the rest after a part 1.
  auto prefetch = [&](uint32_t st_off, int part = 0) {
    const uint32_t st = lds_base + st_off;
    const bool kcopy = !RING || pc_loc < ksteps;
    if (part == 1) {
      if constexpr (KM != kAligned8) {
        uint32_t wv[kCB];
#pragma unroll
        for (int q = 0; q < kCB; ++q) wv[q] = pc_wv + q * row8;
        if (KM == kAligned16 && (int64_t)pc_loc * kTileK + k_lane + 8 > K) {
#pragma unroll
          for (int q = 0; q < kCB; ++q) wv[q] = kOobOffset - pc_wso;
        }
        dma_w_tile_part_asm<kCB>(wr, wv, pc_wso, st, lw);
      }
      return;
    }
    if (part == 2) {
      dma_a_tile_asm(ar, ir, pc_aso, pc_iso, va, vi, st, la, li);
    } else if (kcopy) {
      if constexpr (KM == kAligned8) {
        dma_a_tile_asm(ar, ir, pc_aso, pc_iso, va, vi, st, la, li);
        dma_w_tile_dword<kWaves>(wr, N, K, pc_n0, (int64_t)pc_loc * kTileK, &lds[st_off]);
      } else {
        uint32_t wv[kCB];
#pragma unroll
        for (int q = 0; q < kCB; ++q) wv[q] = pc_wv + q * row8;
        // Channel tail (kAligned16): chunks past K point out of the buffer
        // (the range check covers the VGPR and the scalar offset together).
        if (KM == kAligned16 && (int64_t)pc_loc * kTileK + k_lane + 8 > K) {
#pragma unroll
          for (int q = 0; q < kCB; ++q) wv[q] = kOobOffset - pc_wso;
        }
        dma_kstep_asm<kCB>(wr, ar, ir, wv, pc_wso, pc_aso, pc_iso, va, vi, st, lw, la, li);
      }
    } else {
      if constexpr (RING) dma_lora_tile_asm<kCB, kOps>(tr, br, pc_tb0, rsteps, pc_loc - ksteps, N, r, pc_n0, st);
    }
    if constexpr (PFW) {
      constexpr int kPfDist = 4;
      const int tgt = pc_loc + kPfDist;
      if (((pc_loc + pc_i) & 7) == wave && tgt < ksteps) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(pf_r0 * (uint32_t)(2 * K) + (uint32_t)tgt * (2u * kTileK));
        const int64_t left = N - (int64_t)pf_r0;
        const uint32_t lim = left < 32 ? (uint32_t)(left > 0 ? left : 0) : 32u;
        const uint32_t voff = (uint32_t)lane < lim ? base + (uint32_t)lane * (uint32_t)(2 * K) : kOobOffset;
        l2_probe_asm(wr, voff, lds_base + (uint32_t)T::kProbeOff + 256u * (uint32_t)wave);
      }
    }
    if (pc_loc + 1 < spt) {
      ++pc_loc;
      pc_wso += 2u * kTileK;
      pc_aso += 8192u;
      pc_iso += 1024u;
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
    dma_scale_asm(sr, (uint32_t)(tm * kTileM * 4), lds_base + kScaleOff + (uint32_t)(i & 1) * 1024u, vi);
  };

  const char* b_base0 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(0);
  const char* b_base1 = &lds[0] + wn * kCB * 2048 + frag_lane_offset(1);
  const char* a_base = &lds[0] + kAStageOff + 16 * lane + wm * 8192;
  const char* i_base = &lds[0] + kIStageOff + 16 * lane + wm * 1024;

  // Stages by LDS byte offset: o_cur is the step's stage, o_nxt the next
  // one, o_pf the one after (in flight); the three rotate after each step.
  uint32_t o_cur = 0, o_nxt = kStageBytes, o_pf = 2 * kStageBytes;
  auto rotate = [&]() {
    const uint32_t t = o_cur;
    o_cur = o_nxt;
    o_nxt = o_pf;
    o_pf = t;
  };

  // One barrier per step, once the wave has read all of the step's operands
  // from LDS (the last column block's W fragments included) and waited for
  // its own copies of the next step (only those of the step after may still
  // be in flight).  After it, stage o_nxt is complete for every wave and
  // stage o_cur is free: it is refilled with the step three ahead, at once
  // while the step's last MFMAs run (a copy then has two steps to land), or
  // by the second wavefront of each SIMD after an early column block of the
  // next k-step (late refill: still before the next barrier, so the waits
  // count the same operations).
  // after_stores: the previous tile's output stores were issued after the
  // awaited copies and may still be in flight (vmcnt counts them too).
  // Epilogue staging: 1 row block per pass (16 rows x store_pitch per
  // wavefront: 18 KiB for 8 wavefronts, the stage's A and position
  // regions) in the ring shapes with 16-byte copies, else 2 per pass.
  constexpr bool kEarlyW = RING && KM != kAligned8;
  constexpr int kPRB = kEarlyW ? 1 : 2;
  constexpr int kStoreOps = store_passes_ops<kRB, kCB, kPRB>();
  static_assert(2 * kOps + kStoreOps < 64, "vmcnt field is 6 bits");
  auto step_barrier = [&](bool after_stores) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (after_stores) wait_vm<kOps + kStoreOps>();
    else wait_vm<kOps>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The refill of the stage just consumed, plus the next tile's scales on a
  // tile's first step.
  auto refill = [&](int64_t scales_for) {
    __builtin_amdgcn_sched_barrier(0);
    prefetch(o_cur);
    if (scales_for >= 0) copy_scales(scales_for);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Operands a k-step starts with: the position fields, the 8 A fragments
  // and the first column block of W, read from the stage at offset o.
  u32x4 iw, bq0, bq1;
  bf16x8 af[kRB];
  auto load_first = [&](uint32_t o) {
    iw = *reinterpret_cast<const u32x4*>(i_base + o);
    bq0 = *reinterpret_cast<const u32x4*>(b_base0 + o);
    bq1 = *reinterpret_cast<const u32x4*>(b_base1 + o);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      af[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + o + rb * 1024));
  };

  f32x4 acc[kRB][kCB];

  // Late refill.  A refill burst holds its wavefront in issue while the
  // copy path drains; when both wavefronts of a SIMD (waves w and w + 4)
  // burst after the same barrier, its matrix core idles.  Waves 4-7
  // therefore issue the refill of the stage a k-step consumed after column
  // block kLateCb of the next k-step: 1 with 256-column tiles, 0 with
  // 192-column tiles (each measured 3-4 % and 2.5 % faster than no late
  // refill; the other choice of block was slower for either width).
  constexpr int kLateCb = CB == 4 ? 1 : 0;
  const bool late_wave = wave >= 4;
  bool late_pending = false;
  uint32_t late_stage = 0;

  // One k-step: 8 CB structured-sparse MFMAs, the W fragments (two 16-byte
  // halves per lane, swizzled tile) read one column block ahead.  The
  // position fields of row blocks 2j and 2j+1 share a 32-bit word (abid).
  // The last column block runs after the step's barrier, together with the
  // reads of the next step's first operands and the refill (deferred to the
  // epilogue on a tile's last step, whose stage the epilogue uses; late, if
  // late_ok, for waves 4-7: the next step is then a k-step of the tile, which
  // issues it).
  auto kstep = [&](int64_t scales_for, bool after_stores, bool defer, bool late_ok) {
    const char* s0 = b_base0 + o_cur;
    const char* s1 = b_base1 + o_cur;
    const uint32_t on = o_nxt;
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
        if (cb == kLateCb && late_pending) {
          __builtin_amdgcn_sched_barrier(0);
          prefetch(late_stage);
          __builtin_amdgcn_sched_barrier(0);
          late_pending = false;
        }
      } else {
        step_barrier(after_stores);
        const u32x4 iw_cur = iw;
        iw = *reinterpret_cast<const u32x4*>(i_base + on);
        bq0 = *reinterpret_cast<const u32x4*>(b_base0 + on);
        bq1 = *reinterpret_cast<const u32x4*>(b_base1 + on);
#pragma unroll
        for (int rb = 0; rb < kRB; rb += 2) {
          acc[rb][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb], bf, acc[rb][cb], (int)iw_cur[rb / 2], 0, 0);
          acc[rb + 1][cb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[rb + 1], bf, acc[rb + 1][cb], (int)iw_cur[rb / 2], 0, 1);
          af[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + on + rb * 1024));
          af[rb + 1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_base + on + (rb + 1) * 1024));
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
        if (!defer) {
          if (late_wave && late_ok) {
            late_pending = true;
            late_stage = o_cur;
          } else {
            refill(scales_for);
          }
        }
      }
    }
    if (defer && scales_for >= 0) copy_scales(scales_for);
    rotate();
  };

  // One LoRA step: for each half (hi, lo) of alpha T / s, 8 row fragments
  // and CB B fragments from LDS, 8 CB dense MFMAs; the barrier comes once
  // the lo half is read, the refill behind it.
  auto lstep = [&](bool defer) {
    const char* st = &lds[0] + o_cur + 16 * lane;
    bf16x8 bfr[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
      bfr[cb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + T::kLoraBOff + (wn * kCB + cb) * 1024));
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      bf16x8 ta[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        ta[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + ((wm * kRB + rb) * 2 + hl) * 1024));
      if (hl == 1) {
        step_barrier(false);
        if (!defer) refill(-1);
      }
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta[rb], bfr[cb], acc[rb][cb], 0, 0, 0);
    }
    rotate();
  };

  // Prologue: the first tile's scales, then the copies of steps 0, 1 and 2;
  // wait for step 0's and read its first operands.
  copy_scales(0);
  prefetch(0);
  prefetch(kStageBytes);
  prefetch(2 * kStageBytes);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<2 * kOps>();
  barrier_no_fence();
  __builtin_amdgcn_sched_barrier(0);
  load_first(0);

  for (int i = 0; i < my_tiles; ++i) {
    int64_t tm, tn;
    tile_coords_of((int64_t)blockIdx.x + (int64_t)i * G, tiles_m, tiles_n, tm, tn);
    const int64_t n0 = tn * kTileN;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) acc[rb][cb] = (f32x4){0, 0, 0, 0};

    // One step per iteration, the stage a runtime offset: unrolled copies
    // of the step get different accumulator registers from the register
    // allocator, and the copies between them wait on the matrix pipeline.
    // The first step also copies the next tile's scales; the tile's last
    // step leaves its refill to the epilogue.
    const int64_t next_scales = i + 1 < my_tiles ? i + 1 : -1;
    const bool after_stores = i > 0 && N % 8 == 0;
    // Late refills only from the middle k-steps, whose next step is a k-step
    // of the tile: none is pending across a LoRA step or the epilogue.
    kstep(next_scales, after_stores, lsteps == 0 && ksteps == 1, false);
#pragma nounroll
    for (int ks = 1; ks < ksteps - 1; ++ks) kstep(-1, false, false, true);
    if (ksteps > 1) kstep(-1, false, lsteps == 0, false);
    if constexpr (RING) {
      for (int g = 0; g < lsteps; ++g) lstep(g == lsteps - 1);
    }

    // Epilogue.  Every wave has passed the last step's barrier, so the
    // stage that step consumed (o_pf after the rotation) is free: the tile
    // is staged through it before the deferred refill, or, when that refill
    // is a k-step (the ring shapes with 16-byte copies), through its A
    // region only while the refill's W tile goes out first into its W
    // region (early W: the copy path works during the epilogue's conversion
    // and LDS passes; 0.3-1.1 % faster at the shapes with several tiles per
    // workgroup, outputs bit-identical).  The next stage is complete and the
    // one after is in flight.
    __builtin_amdgcn_sched_barrier(0);
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
    // scales were copied on the previous tile's first step, or in the
    // prologue.)
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
    const bool early_w = kEarlyW && N % 8 == 0 && pc_loc < ksteps;
    if (N % 8 == 0) {
      if (early_w) {
        // The deferred refill's W tile goes out now, into the W region of
        // the free stage; the tile is staged through its A region.
        __builtin_amdgcn_sched_barrier(0);
        prefetch(o_pf, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      char* region = &lds[0] + o_pf + (kEarlyW ? kAStageOff : 0) + wave * (16 * kPRB * store_pitch<kCB>());
      store_tile_via_lds_passes<kRB, kCB, kPRB>(acc, region, y, M, N, m0, n0 + wn * kWaveN);
    } else {
      store_acc_bf16<kRB, kCB>(acc, y, M, N, m0, n0 + wn * kWaveN);
    }
    // Every wave is done with the staging area: the deferred refill (its
    // A tile and position fields only, after an early W) goes there.  The
    // next tile starts from stage o_cur, complete since the last step's
    // barrier.  The vmcnt waits count the same operations either way: the
    // refill's copies, split or not, and the stores come before the next
    // tile's first barrier.
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    prefetch(o_pf, early_w ? 2 : 0);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < my_tiles) load_first(o_cur);
  }
  // Drain the remaining (redundant) copies before the workgroup's LDS is
  // released.
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
}

}  // namespace

namespace {

template <int CB>
hipError_t launch_sparse_gemm_t(const u32x4* xv, const uint16_t* xi, const float* s, const u32x4* t,
                                const uint16_t* w, const uint16_t* lora_b, int64_t M, int64_t N, int64_t K,
                                int64_t r, int64_t kpairs, int64_t rsteps, uint16_t* y, int64_t cus,
                                hipStream_t stream, bool prefetch_w) {
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + Tile<CB>::kTileNc - 1) / Tile<CB>::kTileNc);
  // One persistent workgroup per CU (the LDS allows one), at most one per tile.
  const dim3 grid((unsigned)(tiles < cus ? tiles : cus)), block(kThreads);
  // The k loop runs over the padded K (a multiple of 128): full-K mode
  // needs K itself to be one.
  const bool ring = r % 8 == 0;
  using Kern = decltype(&sparse_gemm_kernel<kFullK, true, CB, false>);
  Kern k = nullptr;
  if (K % 128 == 0)
    k = !ring ? &sparse_gemm_kernel<kFullK, false, CB, false>
        : prefetch_w ? &sparse_gemm_kernel<kFullK, true, CB, true> : &sparse_gemm_kernel<kFullK, true, CB, false>;
  else if (K % 8 == 0)
    k = !ring ? &sparse_gemm_kernel<kAligned16, false, CB, false>
        : prefetch_w ? &sparse_gemm_kernel<kAligned16, true, CB, true> : &sparse_gemm_kernel<kAligned16, true, CB, false>;
  else if constexpr (CB == 4) k = &sparse_gemm_kernel<kAligned8, false, CB, false>;
  if (k == nullptr) return hipErrorInvalidValue;   // K % 8 == 4 takes 256-column tiles
  return launch(k, grid, block, stream, xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y);
}

}  // namespace

int sparse_gemm_tile_n(int64_t M, int64_t N, int64_t K, int compute_units) {
  // 192-column tiles when they fill the CUs in fewer tile rounds, weighed by
  // their cost relative to a 256-column tile: the kernel is bound by its
  // operand copies, 42 KiB per k-step against 50 KiB (0.84).
  if (K % 8 != 0) return 256;
  const int64_t cus = compute_units > 0 ? compute_units : 1;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM;
  auto rounds = [&](int64_t tn) { return (tiles_m * ((N + tn - 1) / tn) + cus - 1) / cus; };
  return rounds(192) * 84 < rounds(256) * 100 ? 192 : 256;
}

hipError_t launch_sparse_gemm(const void* workspace, const uint16_t* w, const uint16_t* lora_b,
                              int64_t M, int64_t N, int64_t K, int64_t r, uint16_t* y,
                              int compute_units, hipStream_t stream, int tile_n, bool prefetch_w) {
  const WsLayout L = ws_layout(M, K, r);
  const char* ws = static_cast<const char*>(workspace);
  const u32x4* xv = reinterpret_cast<const u32x4*>(ws + L.off_xv);
  const uint16_t* xi = reinterpret_cast<const uint16_t*>(ws + L.off_xi);
  const float* s = reinterpret_cast<const float*>(ws + L.off_s);
  const u32x4* t = reinterpret_cast<const u32x4*>(ws + L.off_t);
  const int64_t kpairs = L.kp / 128, rsteps = L.rp / 32;
  const int64_t cus = compute_units > 0 ? compute_units : 1;
  if (tile_n == 0) tile_n = sparse_gemm_tile_n(M, N, K, compute_units);
  if (tile_n == 192 && K % 8 == 0)
    return launch_sparse_gemm_t<3>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y, cus, stream, prefetch_w);
  return launch_sparse_gemm_t<4>(xv, xi, s, t, w, lora_b, M, N, K, r, kpairs, rsteps, y, cus, stream, prefetch_w);
}

}  // namespace rtl
