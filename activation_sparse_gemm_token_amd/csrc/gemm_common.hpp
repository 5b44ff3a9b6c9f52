// Pieces shared by the structured-sparse and the dense GEMM kernels.
//
// Both kernels compute a 256 x 256 output tile per workgroup and stream
// their operands through a ring of LDS stages in 64-deep k-steps, filled
// by direct global -> LDS copies (buffer_load ... lds).  Both run 8
// wavefronts of 128 x 64 (two per SIMD: one wavefront alone cannot issue LDS
// reads fast enough to feed the matrix core, and idles it through its own
// waits).  The helpers below are
// templated on the number of wavefronts WAVES that share a tile copy and on
// the wavefront's block counts RB x CB (16 x 16 blocks).
#pragma once

#include "rtl_common.hpp"

namespace rtl {

constexpr int kTileM = 256, kTileN = 256, kTileK = 64;
constexpr int kTileBytes = kTileN * kTileK * 2;              // one 256 x 64 bf16 tile: 32 KiB

// How channel tails are handled.  kFullK: every k-step lies inside K (no
// guard, the common case); kAligned16: rows are 16-byte aligned and the last
// k-step is partial (16-byte copies, guarded per chunk); kAligned8: K % 8 ==
// 4, rows are only 8-byte aligned (4-byte copies, guarded per pair).
enum KMode { kFullK = 0, kAligned16 = 1, kAligned8 = 2 };

// A 256-row x 64-channel bf16 tile in LDS (the W tile, and the X tile of
// the dense kernel): row-major, 128 bytes per row, with the 16-byte chunk c
// (channels 8c .. 8c + 7) of row n stored in slot c ^ (n & 7) of the row.
// The copy then reads whole 128-byte lines of the row-major source (8 lanes
// per row), and a fragment read -- 16 rows at one chunk index -- spreads
// over all LDS banks.
//
// Copy: wavefront v moves rows (256 / WAVES) v + [0, 256 / WAVES), 8 rows
// per instruction; lane l fills LDS slot l % 8 of row l / 8 of its 8 (the
// DMA writes lane l's 16 bytes to M0 + 16 l) with source chunk
// (l % 8) ^ (l / 8).  Byte offsets (at channel 0) are one per-lane base
// plus a uniform 8-row step, so one VGPR stays live; rows past the end of
// the tensor lie past its end and read as zeros (the row is in the VGPR
// offset, which the buffer range check covers).
struct WTileOffsets {
  uint32_t base;                  // VGPR
  uint32_t row8;                  // uniform: bytes of 8 rows
  int32_t k_lane;                 // 8 ((l % 8) ^ (l / 8))
  __device__ __forceinline__ uint32_t off(int i) const { return base + (uint32_t)i * row8; }
};

template <int WAVES>
__device__ __forceinline__ WTileOffsets w_tile_offsets(int64_t K, int64_t n0) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WTileOffsets o;
  o.k_lane = 8 * ((lane & 7) ^ (lane >> 3));
  o.base = (uint32_t)(((n0 + (256 / WAVES) * wave + (lane >> 3)) * K + o.k_lane) * 2);
  o.row8 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * K * 2));
  return o;
}

// Per-lane byte offset, inside a 16-row block of such a tile, of the lane's
// fragment for k-half h (channels 32 h + 8 (l / 16) + [0, 8) of row l % 16):
// the operand order of v_mfma_f32_16x16x32_bf16 (both operands) and the
// two halves of v_smfmac_f32_16x16x64_bf16's B operand.  Row block b adds
// 2048 b.
__device__ __forceinline__ uint32_t frag_lane_offset(int h) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)((lane & 15) * 128 + (((4 * h + (lane >> 4)) ^ (lane & 7)) << 4));
}

// The tile copy at channel k0 (K % 8 == 0) as one inline-asm block of
// 32 / WAVES buffer_load_dwordx4 ... lds instructions.  The compiler does
// not see these loads, so it never inserts vmcnt waits for them (with the
// builtin it sometimes cannot prove that a copy into one stage does not
// alias reads of another, and drains all loads); the caller accounts for
// them with explicit vmcnt waits.  The block has no output registers -- the
// data goes to LDS -- and writes only M0, which it saves and restores; it
// uses no instruction that sets SCC.  s_nop 4 covers a VALU write of an
// SGPR operand right before the block, and one wait state follows every M0
// write before the copy that reads it.  With guard_k, chunks past K are
// pointed out of the buffer and arrive as zeros.
template <int WAVES>
__device__ __forceinline__ void dma_w_tile_asm(__amdgpu_buffer_rsrc_t wr, const WTileOffsets& o, int64_t K,
                                               int64_t k0, uint32_t lds_stage_addr, bool guard_k) {
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 wavefronts share a tile copy");
  constexpr int NI = 32 / WAVES;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(k0 * 2));
  const bool chunk_ok = !guard_k || k0 + o.k_lane + 8 <= K;
  uint32_t v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) v[i] = chunk_ok ? o.off(i) : kOobOffset - soff;
  // LDS byte address of instruction i: stage + 128 ((256 / WAVES) wave + 8 i).
  // All are computed outside the block, which then only moves them into M0
  // (s_mov does not touch SCC).
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_stage_addr + 128u * (256 / WAVES) * (uint32_t)wave);
  uint32_t saved;
  if constexpr (NI == 8) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[l0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v0], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v1], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l2]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v2], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l3]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v3], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l4]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v4], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l5]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v5], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l6]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v6], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l7]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v7], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]), [v3] "v"(v[3]), [v4] "v"(v[4]), [v5] "v"(v[5]),
          [v6] "v"(v[6]), [v7] "v"(v[7]), [rs] "s"(wr), [so] "s"(soff), [l0] "s"(l0), [l1] "s"(l0 + 0x400u),
          [l2] "s"(l0 + 0x800u), [l3] "s"(l0 + 0xc00u), [l4] "s"(l0 + 0x1000u), [l5] "s"(l0 + 0x1400u),
          [l6] "s"(l0 + 0x1800u), [l7] "s"(l0 + 0x1c00u)
        : "memory");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[l0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v0], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v1], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l2]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v2], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l3]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v3], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]), [v3] "v"(v[3]), [rs] "s"(wr), [so] "s"(soff),
          [l0] "s"(l0), [l1] "s"(l0 + 0x400u), [l2] "s"(l0 + 0x800u), [l3] "s"(l0 + 0xc00u)
        : "memory");
  }
  (void)saved;
}

// Tile copy for K % 8 == 4 (rows only 8-byte aligned): 128 / WAVES dword
// DMAs per thread through the builtin, which the compiler tracks (and
// drains before later LDS reads -- slow, but this mode only serves odd
// channel counts).  Instruction b of wavefront v fills rows
// (256 / WAVES) v + 2 b + [0, 2); DMA lane j writes dword j % 4 of slot
// (j % 32) / 4 of row j / 32, so the LDS layout matches the 16-byte copy.
template <int WAVES>
__device__ __forceinline__ void dma_w_tile_dword(__amdgpu_buffer_rsrc_t wr, int64_t N, int64_t K, int64_t n0,
                                                 int64_t k0, char* lds_stage) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int b = 0; b < 128 / WAVES; ++b) {
    const int row = (256 / WAVES) * wave + 2 * b + (lane >> 5);
    const int chunk = ((lane & 31) >> 2) ^ (row & 7);
    const int64_t n = n0 + row;
    const int64_t k = k0 + 8 * chunk + 2 * (lane & 3);
    const uint32_t voff = (k + 2 <= K && n < N) ? (uint32_t)((n * K + k) * 2) : kOobOffset;
    char* dst = lds_stage + ((256 / WAVES) * wave + 2 * b) * 128;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(dst), 4, voff, 0, 0, 0);
  }
}

// Workgroup barrier without the release fence of __syncthreads(), whose
// "vmcnt(0)" would also drain the copies of later stages still in flight.
// The asm statement is a full compiler memory barrier; the caller waits
// explicitly for the data the barrier publishes.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Waits until at most n vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup id i runs on XCD i % 8), and each XCD has its own L2.  The id
// is first renumbered so that every XCD owns a contiguous range of tiles,
// then that range is walked in groups of kGroupN tile columns, column
// fastest, so the ~32 tiles an XCD runs at once form an 8 x 4 block: per
// k-step they share 8 A slices and 4 W slices in L2 instead of 1 and 32.
constexpr int kXcds = 8;
constexpr int kGroupN = 4;

// Tile of ordinal `id` (the workgroup id, or a persistent workgroup's
// virtual id blockIdx.x + i * gridDim.x, which runs on the same XCD).
__device__ __forceinline__ void tile_coords_of(int64_t id, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                               int64_t& tn) {
  const int64_t total = tiles_m * tiles_n;
  const int64_t xcd = id % kXcds, local = id / kXcds;
  const int64_t per = total / kXcds, extra = total % kXcds;
  const int64_t lin = xcd * per + (xcd < extra ? xcd : extra) + local;   // bijection on [0, total)
  const int64_t per_group = (int64_t)kGroupN * tiles_m;
  const int64_t g = lin / per_group;
  const int64_t first_n = g * kGroupN;
  const int64_t gw = tiles_n - first_n < kGroupN ? tiles_n - first_n : kGroupN;
  const int64_t in = lin - g * per_group;
  tm = in / gw;
  tn = first_n + in % gw;
}

__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  tile_coords_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
}

// Stores a wavefront's (16 RB) x (16 CB) fp32 accumulators as bf16, one
// element per lane and store (any N).
template <int RB, int CB>
__device__ __forceinline__ void store_acc_bf16(const f32x4 (&acc)[RB][CB], uint16_t* __restrict__ y,
                                               int64_t M, int64_t N, int64_t m0, int64_t n0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int64_t n = n0 + 16 * cb + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const uint32_t p = cvt_pk_bf16(acc[rb][cb][i], acc[rb][cb][i + 1]);
        const int64_t m = m0 + 16 * rb + 4 * (lane >> 4) + i;
        if (m < M && n < N) y[m * N + n] = (uint16_t)p;
        if (m + 1 < M && n < N) y[(m + 1) * N + n] = (uint16_t)(p >> 16);
      }
    }
  }
}

// Epilogue store through LDS.  Each wavefront writes its (16 RB) x (16 CB)
// tile as bf16 into its own LDS region (row pitch 32 CB + 16 bytes: 16-byte
// aligned rows, and the four row groups of one write fall on different
// banks), then reads it back 16 bytes per lane along rows and issues
// coalesced 16-byte buffer stores (whole rows of the tile) instead of
// scattered 2-byte stores.  The caller must have drained every copy and
// passed a barrier, so that the LDS ring is free (store_lds_bytes).
// Requires N % 8 == 0 (a chunk of 8 columns is all inside or all outside
// Y); chunks past M or N are pointed out of range, and the whole offset is
// in the VGPR operand.
template <int CB>
constexpr int store_pitch() { return 32 * CB + 16; }

template <int RB, int CB>
constexpr int store_lds_bytes(int waves) { return waves * 16 * RB * store_pitch<CB>(); }

// Writes the staged region (16 ROWS rows of 2 CB 16-byte chunks at row pitch
// store_pitch<CB>()) to Y as coalesced 16-byte buffer stores, whole rows of
// the tile per store.
template <int ROWS16, int CB>
__device__ __forceinline__ void flush_staged_region(const char* region, uint16_t* __restrict__ y, int64_t M,
                                                    int64_t N, int64_t m0, int64_t n0) {
  constexpr int kPitch = store_pitch<CB>();
  constexpr int kChunks = 2 * CB;                  // 16-byte chunks per row
  constexpr int kRowsPerPass = 64 / kChunks;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, M * N * 2);
  const int sub_row = lane / kChunks, chunk = lane % kChunks;
  const int64_t col = n0 + 8 * chunk;
  const bool col_ok = col + 8 <= N;
  const uint32_t lane_off = (uint32_t)(((m0 + sub_row) * N + col) * 2);
  const uint32_t pass_bytes = (uint32_t)(kRowsPerPass * N * 2);
#pragma unroll
  for (int it = 0; it < 16 * ROWS16 / kRowsPerPass; ++it) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + (kRowsPerPass * it + sub_row) * kPitch + 16 * chunk);
    const bool ok = col_ok && m0 + kRowsPerPass * it + sub_row < M;
    const uint32_t voff = ok ? lane_off + (uint32_t)it * pass_bytes : kOobOffset;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), yr,
                                           voff, 0, 0);
  }
}

template <int RB, int CB>
__device__ __forceinline__ void store_tile_via_lds(const f32x4 (&acc)[RB][CB], char* lds_base,
                                                   uint16_t* __restrict__ y, int64_t M, int64_t N,
                                                   int64_t m0, int64_t n0) {
  constexpr int kPitch = store_pitch<CB>();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char* region = lds_base + wave * 16 * RB * kPitch;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int row = 16 * rb + 4 * (lane >> 4) + i, col = 16 * cb + (lane & 15);
        const uint32_t p = cvt_pk_bf16(acc[rb][cb][i], acc[rb][cb][i + 1]);
        *reinterpret_cast<uint16_t*>(region + row * kPitch + 2 * col) = (uint16_t)p;
        *reinterpret_cast<uint16_t*>(region + (row + 1) * kPitch + 2 * col) = (uint16_t)(p >> 16);
      }
  // Only this wavefront reads its region back: a wave-local LDS wait suffices.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  flush_staged_region<RB, CB>(region, y, M, N, m0, n0);
}

// Vector-memory operations (buffer stores) store_tile_via_lds_passes
// issues per wavefront: per pass, the 16 PRB x 2 CB chunks of 16 bytes,
// 64 per store.
template <int RB, int CB, int PRB>
constexpr int store_passes_ops() { return (RB / PRB) * ((16 * PRB * 2 * CB + 63) / 64); }

// The same store in passes of PRB row blocks through a smaller region
// (16 PRB rows x store_pitch<CB>() bytes per wavefront at `region`), for a
// persistent kernel whose ring keeps the next tile's copies in flight.  The
// read-back walks the pass's (row, 16-byte chunk) items 64 at a time, so any
// CB works (2 CB chunks per row need not divide 64).
template <int RB, int CB, int PRB>
__device__ __forceinline__ void store_tile_via_lds_passes(const f32x4 (&acc)[RB][CB], char* region,
                                                          uint16_t* __restrict__ y, int64_t M, int64_t N,
                                                          int64_t m0, int64_t n0) {
  static_assert(RB % PRB == 0, "whole passes");
  constexpr int kPitch = store_pitch<CB>();
  constexpr int kChunks = 2 * CB;                  // 16-byte chunks per row
  constexpr int kItems = 16 * PRB * kChunks;       // per pass
  constexpr int kIters = (kItems + 63) / 64;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, M * N * 2);
#pragma unroll
  for (int pass = 0; pass < RB / PRB; ++pass) {
#pragma unroll
    for (int rr = 0; rr < PRB; ++rr)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int row = 16 * rr + 4 * (lane >> 4) + i, c = 16 * cb + (lane & 15);
          const uint32_t p = cvt_pk_bf16(acc[pass * PRB + rr][cb][i], acc[pass * PRB + rr][cb][i + 1]);
          *reinterpret_cast<uint16_t*>(region + row * kPitch + 2 * c) = (uint16_t)p;
          *reinterpret_cast<uint16_t*>(region + (row + 1) * kPitch + 2 * c) = (uint16_t)(p >> 16);
        }
    // Only this wavefront reads its region back; LDS operations of one
    // wavefront execute in order, so the next pass's writes cannot overtake
    // these reads.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t mp = m0 + 16 * PRB * pass;
    if constexpr (64 % kChunks == 0) {
      // Whole rows per store: each lane keeps its chunk (column) throughout.
      constexpr int kRowsPerPass = 64 / kChunks;
      const int sub_row = lane / kChunks, chunk = lane % kChunks;
      const int64_t col = n0 + 8 * chunk;
      const bool col_ok = col + 8 <= N;
      const uint32_t lane_off = (uint32_t)(((mp + sub_row) * N + col) * 2);
      const uint32_t pass_bytes = (uint32_t)(kRowsPerPass * N * 2);
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(region + (kRowsPerPass * it + sub_row) * kPitch + 16 * chunk);
        const bool ok = col_ok && mp + kRowsPerPass * it + sub_row < M;
        const uint32_t voff = ok ? lane_off + (uint32_t)it * pass_bytes : kOobOffset;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v),
                                               yr, voff, 0, 0);
      }
    } else {
      const uint32_t pass_base = (uint32_t)(mp * N * 2), n2 = (uint32_t)(N * 2);
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int item = 64 * it + lane;
        const int row = item / kChunks, chunk = item % kChunks;
        const bool in = item < kItems;
        const u32x4 v = *reinterpret_cast<const u32x4*>(region + (in ? row * kPitch + 16 * chunk : 0));
        const int64_t col = n0 + 8 * chunk;
        const bool ok = in && col + 8 <= N && mp + row < M;
        const uint32_t voff = ok ? pass_base + (uint32_t)row * n2 + (uint32_t)col * 2u : kOobOffset;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v),
                                               yr, voff, 0, 0);
      }
    }
  }
}

}  // namespace rtl
