// Pre-pass of rtl_sparse_linear: the one kernel that reads X.
//
// For every token it makes the 2:4 pattern decision and Top-K selection
// (qingkeai RT-Lynx article, sections 01 and 04), measures the kept and
// pruned L1 mass and forms the compensation scale s (ai-feeds summary,
// 方法 / 核心模块 1; qingkeai article, section 03.1), compresses the kept
// values together with their 2-bit positions directly into the register
// order of gfx950's v_smfmac_f32_16x16x64_bf16 A operand ("layout
// generation", qingkeai article, section 04), and computes the LoRA-down
// product of the pruned residual (qingkeai article, section 03.2):
//
//   T = (X - S(X)) A^T = ((1-M)*X) A^T + (1 - s) * ((M*X) A^T)
//
// In the generic kernel both terms are 2:4-sparse products of exact input
// words, so they run on the structured-sparse matrix cores with the kept and
// the pruned halves of each group, and no cancellation happens in fp32; the
// DMA-streamed kernel (r <= 64) forms X A^T - s (M*X) A^T instead (dense
// MFMAs on the input words as loaded, no pruned operand to gather; see
// there).  alpha*T/s is stored as a
// bf16 hi/lo pair in the dense 16x16x32 A-operand order: divided by the
// token's scale (s >= 1), so that the GEMM can accumulate the LoRA-up
// product into the same fp32 accumulators as the sparse product and apply
// s once at the end, Y = s (S(X) W^T + (alpha T / s) B^T).
//
// Selection happens here, once per element, and not in the GEMM prologue:
// there it would be repeated for every N tile, and its VALU cost (about 48
// lane operations per group of 4, from the instruction counters) exceeds
// the structured-sparse MFMA time of the tile.
//
// Grid: one workgroup of 8 wavefronts per 16-token block; wavefront w covers
// a contiguous range of 128-channel k-pairs.  Lane l handles token l % 16 and
// the 16 channels (4 groups) starting at 16 * (l / 16) of each 64-channel
// k-step, which is exactly the lane's share of the A operand.
#include "rtl_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

constexpr int kWaves = 8;

// Four groups (16 channels) of one lane: returns the kept and pruned operand
// words and their 16-bit index fields.
struct Quad {
  u32x4 kept, pruned;
  uint32_t kcode, pcode;
};

__device__ __forceinline__ void select_quad(const uint32_t (&w)[8], Quad& q, float& lk, float& lp,
                                            bool fold = false, u32x4* kept_f = nullptr) {
  q.kcode = 0;
  q.pcode = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t lo = w[2 * g], hi = w[2 * g + 1];
    const Group4 r = rank_group(lo, hi);
    const uint32_t ks = pair_selector_sorted(r.first, r.second);
    const uint32_t ps = pair_selector_sorted(r.third, r.fourth);
    q.kept[g] = __builtin_amdgcn_perm(hi, lo, ks);
    q.pruned[g] = __builtin_amdgcn_perm(hi, lo, ps);
    q.kcode |= code_from_selector(ks) << (4 * g);
    q.pcode |= code_from_selector(ps) << (4 * g);
    lk = add_mag_pair(lk, r.first, r.second);
    lp = add_mag_pair(lp, r.third, r.fourth);
    if (fold) (*kept_f)[g] = fold_group(q.kept[g], r);
  }
}

// The kept half only (the pre-pass with DMA-streamed operands forms the
// LoRA-down from the whole input words instead of the pruned half): kept
// operand words and their 16-bit index field; both L1 sums as above; with
// FOLD also the kept words scaled per group (fold_group).
template <bool FOLD>
__device__ __forceinline__ void select_quad_kept(const uint32_t (&w)[8], u32x4& kept, uint32_t& kcode,
                                                 float& lk, float& lp, u32x4& kept_f) {
  kcode = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t lo = w[2 * g], hi = w[2 * g + 1];
    const Group4 r = rank_group(lo, hi);
    const uint32_t ks = pair_selector_sorted(r.first, r.second);
    kept[g] = __builtin_amdgcn_perm(hi, lo, ks);
    kcode |= code_from_selector(ks) << (4 * g);
    lk = add_mag_pair(lk, r.first, r.second);
    lp = add_mag_pair(lp, r.third, r.fourth);
    if constexpr (FOLD) kept_f[g] = fold_group(kept[g], r);
  }
}

// The loads below go through buffer resources: a guarded element is given
// an offset past the end of the tensor and reads as zero, so no load sits
// behind a branch and the compiler can issue them all before waiting.

// 16 channels k .. k + 15 of one row of X.
template <bool ALIGNED16>
__device__ __forceinline__ void load_quad(__amdgpu_buffer_rsrc_t xr, int64_t row, bool row_ok,
                                          int64_t k, int64_t K, uint32_t (&w)[8]) {
  if constexpr (ALIGNED16) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = row_ok && k + 8 * h + 8 <= K;
      const u32x4 v = buf_load16(xr, ok ? (uint32_t)((row * K + k + 8 * h) * 2) : kOobOffset);
      w[4 * h + 0] = v[0]; w[4 * h + 1] = v[1]; w[4 * h + 2] = v[2]; w[4 * h + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bool ok = row_ok && k + 4 * g + 4 <= K;
      const u32x2 v = buf_load8(xr, ok ? (uint32_t)((row * K + k + 4 * g) * 2) : kOobOffset);
      w[2 * g] = v[0]; w[2 * g + 1] = v[1];
    }
  }
}

// B operand of v_smfmac_f32_16x16x64_bf16 from a row-major [rows, K] bf16
// matrix: lane l takes row n = n0 + l % 16 and the channels
// k0 + 8 (l / 16) + [0, 8) and k0 + 32 + 8 (l / 16) + [0, 8).
template <bool ALIGNED16>
__device__ __forceinline__ bf16x16 load_b_sparse(__amdgpu_buffer_rsrc_t br, int64_t rows, int64_t K,
                                                 int64_t n, int64_t k0, int lane) {
  u32x8 v;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t k = k0 + 32 * h + 8 * (lane >> 4);
    if constexpr (ALIGNED16) {
      const bool ok = n < rows && k + 8 <= K;
      const u32x4 c = buf_load16(br, ok ? (uint32_t)((n * K + k) * 2) : kOobOffset);
      v[4 * h + 0] = c[0]; v[4 * h + 1] = c[1]; v[4 * h + 2] = c[2]; v[4 * h + 3] = c[3];
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bool ok = n < rows && k + 4 * q + 4 <= K;
        const u32x2 c = buf_load8(br, ok ? (uint32_t)((n * K + k + 4 * q) * 2) : kOobOffset);
        v[4 * h + 2 * q] = c[0]; v[4 * h + 2 * q + 1] = c[1];
      }
    }
  }
  return __builtin_bit_cast(bf16x16, v);
}

template <bool ALIGNED16, int NCB, bool FOLD>
__global__ void __launch_bounds__(64 * kWaves)
prepass_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ lora_a,
               int64_t M, int64_t K, int64_t r, float alpha,
               u32x4* __restrict__ xv, uint16_t* __restrict__ xi, float* __restrict__ s_out,
               u32x4* __restrict__ t_out, int64_t kpairs, int64_t rsteps, int comp, int lora) {
  // NCB = 16-wide column blocks of the LoRA rank covered (0: no LoRA branch).
  constexpr int NT = NCB > 0 ? NCB : 1;
  __shared__ float red_l[kWaves][2][16];
  __shared__ float s_sh[16];
  __shared__ float red_t[NCB > 0 ? kWaves : 1][16][NT * 16 + 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Block mapping: the 8 16-token blocks of a group share 16-byte chunks of
  // the position-field array (2 bytes each), so they are processed on one
  // XCD (workgroup i runs on XCD i % 8), whose L2 merges the partial writes
  // before they reach memory.  Group g runs on XCD g % 8; padding
  // workgroups past the last group exit at once.
  const int64_t ngroups = 2 * ((M + 255) / 256);       // padded rows / 128
  const int64_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int64_t grp_id = 8 * (local / 8) + xcd;
  if (grp_id >= ngroups) return;
  const int64_t mb = 8 * grp_id + local % 8;
  const int64_t row = mb * 16 + (lane & 15);
  const bool row_ok = row < M;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, M * K * 2);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(lora_a, r * K * 2);
  const int64_t ksteps = 2 * kpairs;

  float lk = 0.f, lp = 0.f;
  f32x4 tk[NT], tp[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) { tk[c] = (f32x4){0, 0, 0, 0}; tp[c] = (f32x4){0, 0, 0, 0}; }

  const int64_t p_begin = (int64_t)wave * kpairs / kWaves;
  const int64_t p_end = (int64_t)(wave + 1) * kpairs / kWaves;
  // Software pipeline over the wavefront's k-pairs: the loads of k-pair
  // p + 1 (X and, up to rank 64, the LoRA A operand) are in flight while
  // k-pair p is selected, compressed and multiplied.  Above rank 64 two
  // k-pairs of A operands (2 x 128 registers) do not fit beside the
  // accumulators, nor do two of rank 64 beside the folded words of per-group
  // compensation: A is then loaded in the k-pair's own body, four column
  // blocks at a time.
  constexpr bool kPrefetchA = NCB > 0 && (NCB < 4 || (NCB == 4 && !FOLD));
  constexpr int kChunk = NCB < 4 ? NT : 4;
  uint32_t w0[8], w1[8];
  bf16x16 bA[kPrefetchA ? NT : 1][2];
  auto load_a = [&](int64_t p, int c, bf16x16 (&dst)[2]) {
    const int64_t n = c * 16 + (lane & 15);
    dst[0] = load_b_sparse<ALIGNED16>(ar, r, K, n, 128 * p, lane);
    dst[1] = load_b_sparse<ALIGNED16>(ar, r, K, n, 128 * p + 64, lane);
  };
  auto load_pair = [&](int64_t p) {
    const int64_t k = 128 * p + 16 * (lane >> 4);
    load_quad<ALIGNED16>(xr, row, row_ok, k, K, w0);
    load_quad<ALIGNED16>(xr, row, row_ok, k + 64, K, w1);
    if constexpr (kPrefetchA) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) load_a(p, c, bA[c]);
    }
  };
  if (p_begin < p_end) load_pair(p_begin);
  for (int64_t p = p_begin; p < p_end; ++p) {
    uint32_t x0[8], x1[8];
    bf16x16 b[kPrefetchA ? NT : 1][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) { x0[i] = w0[i]; x1[i] = w1[i]; }
    if constexpr (kPrefetchA) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) { b[c][0] = bA[c][0]; b[c][1] = bA[c][1]; }
    }
    if (p + 1 < p_end) load_pair(p + 1);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t ks0 = 2 * p;
    Quad q0, q1;
    constexpr bool fold = FOLD;        // per-group compensation (comp == kCompGroup)
    u32x4 f0 = (u32x4){0, 0, 0, 0}, f1 = (u32x4){0, 0, 0, 0};
    select_quad(x0, q0, lk, lp, fold, &f0);
    select_quad(x1, q1, lk, lp, fold, &f1);
    const int64_t grp = mb >> 3, sub = mb & 7;
    xv[((grp * ksteps + ks0) * 8 + sub) * 64 + lane] = fold ? f0 : q0.kept;
    xv[((grp * ksteps + ks0 + 1) * 8 + sub) * 64 + lane] = fold ? f1 : q1.kept;
    xi[((grp * ksteps + ks0) * 64 + lane) * 8 + sub] = (uint16_t)q0.kcode;
    xi[((grp * ksteps + ks0 + 1) * 64 + lane) * 8 + sub] = (uint16_t)q1.kcode;
    if constexpr (NCB > 0) {
      // Column blocks c0 .. c0 + kChunk - 1; per block the products go in
      // the same order whichever way A arrived.
#pragma unroll
      for (int c0 = 0; c0 < NCB; c0 += kChunk) {
        bf16x16 bl[kPrefetchA ? 1 : kChunk][2];
        if constexpr (!kPrefetchA) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < kChunk; ++c) load_a(p, c0 + c, bl[c]);
        }
        auto bop = [&](int c, int h) -> const bf16x16& {
          if constexpr (kPrefetchA) return b[c0 + c][h];
          else return bl[c][h];
        };
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          f32x4& k_ = tk[c0 + c];
          f32x4& p_ = tp[c0 + c];
          k_ = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, q0.kept), bop(c, 0), k_, (int)q0.kcode, 0, 0);
          p_ = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, q0.pruned), bop(c, 0), p_, (int)q0.pcode, 0, 0);
          k_ = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, q1.kept), bop(c, 1), k_, (int)q1.kcode, 0, 0);
          p_ = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, q1.pruned), bop(c, 1), p_, (int)q1.pcode, 0, 0);
        }
        if (fold && lora == kLoraResidual) {
          // R's kept part is M*X - S(X): the folded words with their sign
          // flipped (exact) join tk.
#pragma unroll
          for (int c = 0; c < kChunk; ++c) {
            f32x4& k_ = tk[c0 + c];
            k_ = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, f0 ^ 0x80008000u), bop(c, 0), k_, (int)q0.kcode, 0, 0);
            k_ = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, f1 ^ 0x80008000u), bop(c, 1), k_, (int)q1.kcode, 0, 0);
          }
        }
      }
    }
  }

  // Per-token L1 sums: lanes l, l^16, l^32, l^48 share a token; then across
  // wavefronts in a fixed order.
  lk += __shfl_xor(lk, 16, 64);
  lk += __shfl_xor(lk, 32, 64);
  lp += __shfl_xor(lp, 16, 64);
  lp += __shfl_xor(lp, 32, 64);
  if (lane < 16) { red_l[wave][0][lane] = lk; red_l[wave][1][lane] = lp; }
  __syncthreads();
  if (threadIdx.x < 16) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { a += red_l[w][0][threadIdx.x]; b += red_l[w][1][threadIdx.x]; }
    // Per token, or 1 (none; per group: in the operand), or the whole
    // activation's factor, which the statistics pass left in s_out.
    const float s = comp == kCompToken ? (a > 0.f ? (a + b) / a : 1.0f)
                  : comp == kCompTensor ? s_out[mb * 16 + threadIdx.x] : 1.0f;
    s_sh[threadIdx.x] = s;
    s_out[mb * 16 + threadIdx.x] = s;
  }
  if constexpr (NCB > 0) {
    __syncthreads();
    // Accumulator layout of a 16x16 block: lane l holds column l % 16 of rows
    // 4 (l / 16) + i.  T_w = T_pruned + c T_kept per wavefront, then summed
    // over wavefronts in a fixed order: c = 1 - s for the residual (for
    // per-group folding T_kept already holds (M*X - S(X)) A^T: c = 1), 0
    // for the pruned values, 1 for the whole input.
    constexpr bool folded = FOLD;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * (lane >> 4) + i;
        const float ck = lora == kLoraResidual ? (folded ? 1.0f : 1.0f - s_sh[rr]) : lora == kLoraPruned ? 0.0f : 1.0f;
        red_t[wave][rr][c * 16 + (lane & 15)] = tp[c][i] + ck * tk[c][i];
      }
    }
    __syncthreads();
    // Output fragment f = 64 rs + l: token l % 16, rank columns
    // 32 rs + 8 (l / 16) + [0, 8), stored as 4 hi words then 4 lo words;
    // every thread forms words (word j packs columns 2 j and 2 j + 1, each
    // summed over the wavefronts in a fixed order).
    const int nfrag = (int)rsteps * 64;
    uint32_t* const tw = reinterpret_cast<uint32_t*>(t_out);
    for (int q = (int)threadIdx.x; q < 4 * nfrag; q += 64 * kWaves) {
      const int j = q / nfrag, f = q - j * nfrag;
      const int rs = f >> 6, fl = f & 63, rr = fl & 15;
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int col = 32 * rs + 8 * (fl >> 4) + 2 * j + e;
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) a += red_t[w][rr][col];
        v[e] = alpha * a / s_sh[rr];
      }
      const uint32_t h = pack_bf16x2(v[0], v[1]);
      const uint32_t l = pack_bf16x2(v[0] - bf16_lo_to_f32(h), v[1] - bf16_hi_to_f32(h));
      const int64_t o = ((mb * rsteps + rs) * 2) * 64 + fl;
      tw[o * 4 + j] = h;
      tw[(o + 64) * 4 + j] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Pre-pass with DMA-streamed operands (K % 8 == 0, 0 < r <= 64): one
// workgroup of 8 wavefronts (two per SIMD) per 16-token block, wavefront w
// covering an eighth of the k-steps.  Each wavefront streams its own
// operands into its own LDS rings with buffer_load_dwordx4 ... lds (whole
// 128-byte lines, no registers):
//   * X: 16 tokens x 64 channels (2 KiB) per k-step, 2 stages, 1 step ahead;
//   * A: 16 NCB ranks x 64 channels (2 NCB KiB) per k-step, 2 stages, 1 step
//     ahead (L2-resident: every workgroup reads all of A).
// The rings fill the 160 KiB of LDS.  Two wavefronts per SIMD hide each
// other's copy and selection latencies better than one wavefront with deep
// rings (4 wavefronts with X 7 steps and A 2 steps ahead: 12 % slower at
// K = 3072, 10 % at K = 12288; 5, 6 or 7 wavefronts: slower still).
// Both tiles use the swizzled row-major layout of the GEMM's W tile
// (16-byte chunk c of row n in slot c ^ (n & 7)), so the copies read whole
// lines and the fragment reads are conflict-free.  Only the issuing
// wavefront reads its rings, so its own vmcnt wait suffices (no barrier).
// The loads are inline asm, invisible to the compiler; the explicit waits
// count them exactly, together with the stores of xv and xi (the loop's only
// other vector-memory operations).
constexpr int kDWaves = 8;
constexpr int kXStages = 2, kXAhead = 1;
constexpr int kAStages = 2, kAAhead = 1;
static_assert(kXAhead >= kAAhead && kAAhead >= 1 && kAAhead <= 2, "issue order assumed by the waits");
static_assert(kXStages > kXAhead && kAStages > kAAhead, "a stage is refilled only after its step");

// NI 1-KiB copies (8 rows x 128 bytes each): instruction i writes LDS
// lds_addr + 1024 i (through M0) from per-lane source offsets v[i] plus the
// scalar offset soff.  No output registers, M0 saved and restored, one wait
// state between each M0 write and the copy that reads it; the M0 values
// come from SGPRs (no SCC write).
template <int NI>
__device__ __forceinline__ void dma_rows_asm(__amdgpu_buffer_rsrc_t rs, const uint32_t (&v)[NI], uint32_t soff,
                                             uint32_t lds_addr) {
  uint32_t saved;
  if constexpr (NI == 2) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[l0]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v0], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[l1]\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %[v1], %[rs], %[so] offen lds\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [v0] "v"(v[0]), [v1] "v"(v[1]), [rs] "s"(rs), [so] "s"(soff), [l0] "s"(lds_addr),
          [l1] "s"(lds_addr + 0x400u)
        : "memory");
  } else if constexpr (NI == 4) {
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
        : [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]), [v3] "v"(v[3]), [rs] "s"(rs), [so] "s"(soff),
          [l0] "s"(lds_addr), [l1] "s"(lds_addr + 0x400u), [l2] "s"(lds_addr + 0x800u),
          [l3] "s"(lds_addr + 0xc00u)
        : "memory");
  } else {
    static_assert(NI == 8, "2, 4 or 8 row blocks");
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
          [v6] "v"(v[6]), [v7] "v"(v[7]), [rs] "s"(rs), [so] "s"(soff), [l0] "s"(lds_addr),
          [l1] "s"(lds_addr + 0x400u), [l2] "s"(lds_addr + 0x800u), [l3] "s"(lds_addr + 0xc00u),
          [l4] "s"(lds_addr + 0x1000u), [l5] "s"(lds_addr + 0x1400u), [l6] "s"(lds_addr + 0x1800u),
          [l7] "s"(lds_addr + 0x1c00u)
        : "memory");
  }
  (void)saved;
}

// Per-lane source offsets of NI 8-row blocks of a row-major [rows, K] bf16
// matrix at channel k0 (rows row0 + 8 i + l / 8, source chunk
// (l % 8) ^ (l / 8)); rows past `rows` and chunks past K point out of range.
template <int NI>
__device__ __forceinline__ void rows_offsets(int64_t row0, int64_t rows, int64_t K, int64_t k0,
                                             uint32_t (&v)[NI]) {
  const int lane = threadIdx.x & 63;
  const int64_t k = k0 + 8 * ((lane & 7) ^ (lane >> 3));
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t rw = row0 + 8 * i + (lane >> 3);
    v[i] = (rw < rows && k + 8 <= K) ? (uint32_t)((rw * K + k) * 2) : kOobOffset;
  }
}

// Byte offset, inside a swizzled tile (128-byte rows), of chunk c of row n.
__device__ __forceinline__ uint32_t swz(int n, int c) { return (uint32_t)(n * 128 + ((c ^ (n & 7)) << 4)); }

// LoRA-down here: T = X A^T - s (M*X) A^T, the first product by dense
// 16x16x32 MFMAs on the input words as they are, the second by the
// structured-sparse MFMA on the kept half (the same operand the GEMM gets).
// Both accumulate in fp32; the difference loses at most a few units in the
// last place of |X A^T|, far below the rounding of the output.  The L1 sums
// still come from the exact kept and pruned magnitudes.
//
// FULLK (K % 128 == 0, every k-step inside K): the copy and store offsets
// are computed once and advanced by a scalar offset per step; otherwise
// they are recomputed per step with the channel-tail guards.
//
// FOLD (per-group compensation): the stored operand is the kept words scaled
// per group and rounded (fold_group); the LoRA-down subtracts the product of
// that operand.  comp and lora select the other variants at run time.
template <int NCB, bool FULLK, bool FOLD>
__global__ void __launch_bounds__(64 * kDWaves, 1)
prepass_dma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ lora_a,
                   int64_t M, int64_t K, int64_t r, float alpha,
                   u32x4* __restrict__ xv, uint16_t* __restrict__ xi, float* __restrict__ s_out,
                   u32x4* __restrict__ t_out, int64_t ksteps, int64_t rsteps, int comp, int lora) {
  static_assert(NCB == 2 || NCB == 4, "ranks 32 or 64");
  constexpr int kXBytes = 2048;                       // 16 tokens x 128 B
  constexpr int kABytes = NCB * 2048;                 // 16 NCB ranks x 128 B
  constexpr int kWaveBytes = kXStages * kXBytes + kAStages * kABytes;
  constexpr int kXOps = 2, kAOps = 2 * NCB;
  // Reduction arrays, aliased onto the rings after the loop.  T rows of
  // NCB 16 + 4 floats: the accumulator writes (four 16-lane quarters at
  // rows 4 apart) and the epilogue's 32-byte row reads both spread over all
  // LDS banks.
  constexpr int kPitch = NCB * 16 + 4;
  struct Red {
    float l[kDWaves][2][16];
    float s[16];
    float pad[12];
    float t[kDWaves][16][kPitch];
  };
  static_assert((int)sizeof(Red) <= kDWaves * kWaveBytes, "reduction fits in the rings");
  __shared__ __attribute__((aligned(16))) char lds[kDWaves * kWaveBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Same XCD-grouped block mapping as prepass_kernel.
  const int64_t ngroups = 2 * ((M + 255) / 256);
  const int64_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int64_t grp_id = 8 * (local / 8) + xcd;
  if (grp_id >= ngroups) return;
  const int64_t mb = 8 * grp_id + local % 8;
  const int64_t grp = mb >> 3, sub = mb & 7;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, M * K * 2);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(lora_a, r * K * 2);
  // The compressed operand and its position fields of the whole padded
  // workspace (ngroups groups of 8 blocks, ksteps steps).
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(xv, ngroups * ksteps * 8192);
  const __amdgpu_buffer_rsrc_t ir = make_rsrc(xi, ngroups * ksteps * 1024);
  const int ks_begin = (int)(wave * ksteps / kDWaves), ks_end = (int)((wave + 1) * ksteps / kDWaves);
  const int nks = ks_end - ks_begin;                  // uniform per wavefront
  char* const ring = lds + wave * kWaveBytes;
  const uint32_t ring_addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(ring));

  // FULLK: per-lane source offsets at the wavefront's first k-step; a row
  // past the tensor gets 0x80000000, which stays past its end (< 2 GiB)
  // whatever scalar offset is added.
  uint32_t vx[kXOps], va[kAOps];
  if constexpr (FULLK) {
    const int64_t kl = (int64_t)ks_begin * 64 + 8 * ((lane & 7) ^ (lane >> 3));
#pragma unroll
    for (int i = 0; i < kXOps; ++i) {
      const int64_t rw = mb * 16 + 8 * i + (lane >> 3);
      vx[i] = rw < M ? (uint32_t)((rw * K + kl) * 2) : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < kAOps; ++i) {
      const int64_t rw = 8 * i + (lane >> 3);
      va[i] = rw < r ? (uint32_t)((rw * K + kl) * 2) : 0x80000000u;
    }
  }

  // Copies issued together: A of step t_a (if t_a >= 0) first, then X of
  // step t_x, each clamped to the wavefront's last step (a harmless repeat
  // into a stage nobody reads again).  A goes first so that waiting for
  // A(t) -- with in-order completion -- does not also wait for the X copy
  // issued far ahead alongside it.
  auto copy_step = [&](int t_x, int t_a) {
    if (t_a >= 0) {
      const int tc = t_a < nks ? t_a : nks - 1;
      const uint32_t dst = ring_addr + kXStages * kXBytes + (uint32_t)(t_a % kAStages) * kABytes;
      if constexpr (FULLK) {
        dma_rows_asm<kAOps>(ar, va, __builtin_amdgcn_readfirstlane(128u * (uint32_t)tc), dst);
      } else {
        uint32_t v[kAOps];
        rows_offsets<kAOps>(0, r, K, (int64_t)(ks_begin + tc) * 64, v);
        dma_rows_asm<kAOps>(ar, v, 0u, dst);
      }
    }
    const int tc = t_x < nks ? t_x : nks - 1;
    const uint32_t dst = ring_addr + (uint32_t)(t_x % kXStages) * kXBytes;
    if constexpr (FULLK) {
      dma_rows_asm<kXOps>(xr, vx, __builtin_amdgcn_readfirstlane(128u * (uint32_t)tc), dst);
    } else {
      uint32_t v[kXOps];
      rows_offsets<kXOps>(mb * 16, M, K, (int64_t)(ks_begin + tc) * 64, v);
      dma_rows_asm<kXOps>(xr, v, 0u, dst);
    }
  };

  float lk = 0.f, lp = 0.f;
  f32x4 tk[NCB], tx[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) { tk[c] = (f32x4){0, 0, 0, 0}; tx[c] = (f32x4){0, 0, 0, 0}; }

  // Lane l: token l % 16, channels 16 (l / 16) + [0, 16) = chunks 2q, 2q + 1
  // (selection and the structured-sparse operand); chunks q and 4 + q of
  // the token (dense A operands of the two 32-channel halves) and of rank
  // row l % 16 (the B operand halves of both instructions).
  const int tok = lane & 15, q = lane >> 4;
  const uint32_t xo0 = swz(tok, 2 * q), xo1 = swz(tok, 2 * q + 1);
  const uint32_t xd0 = swz(tok, q), xd1 = swz(tok, 4 + q);
  const uint32_t bo0 = swz(tok, q), bo1 = swz(tok, 4 + q);
  // Store offsets: the k-step's 1 KiB of operand words for this 16-token
  // block (lane's 16 bytes) and 16-bit position field; per step they move
  // by 8 KiB and 1 KiB.
  const uint32_t sv0 = (uint32_t)((((grp * ksteps + ks_begin) * 8 + sub) * 64 + lane) * 16);
  const uint32_t si0 = (uint32_t)((((grp * ksteps + ks_begin) * 64 + lane) * 8 + sub) * 2);

  if (nks > 0) {
    // Prologue in the steady-state issue order: step t issues
    // A(t + kAAhead), then X(t + kXAhead); the X copies without an A copy
    // first, then the pairs (A(i), X(kXAhead - kAAhead + i)).
    for (int i = 0; i < kXAhead - kAAhead; ++i) copy_step(i, -1);
    for (int i = 0; i < kAAhead; ++i) copy_step(kXAhead - kAAhead + i, i);
    for (int t = 0; t < nks; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      copy_step(t + kXAhead, t + kAAhead);
      // Wait for step t's copies: A(t) and X(t), whichever came last (X(t)
      // when kXAhead == kAAhead: they go out together, A first).  Younger
      // than it: the X copy issued with A(t) if that was a later step's,
      // the copies of the kAAhead steps after (the last just issued) and
      // the 2 stores (xv, xi) of each step since -- fewer in the first
      // steps.  Vector-memory operations complete in issue order, so the
      // count is exact.
      constexpr int kC = (kXAhead > kAAhead ? kXOps : 0) + kAAhead * (kAOps + kXOps);
      if (t >= kAAhead) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kC + 2 * kAAhead) : "memory");
      else if (t == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kC + 2) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kC) : "memory");
      __builtin_amdgcn_sched_barrier(0);
      const char* xs = ring + (t % kXStages) * kXBytes;
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(xs + xo0);
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(xs + xo1);
      const u32x4 d0 = *reinterpret_cast<const u32x4*>(xs + xd0);
      const u32x4 d1 = *reinterpret_cast<const u32x4*>(xs + xd1);
      const uint32_t w[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      u32x4 kept, kept_f;
      uint32_t kcode;
      select_quad_kept<FOLD>(w, kept, kcode, lk, lp, kept_f);
      const uint32_t so_v = __builtin_amdgcn_readfirstlane(8192u * (uint32_t)t);
      const uint32_t so_i = __builtin_amdgcn_readfirstlane(1024u * (uint32_t)t);
      // The LoRA-down's kept operand: the stored (folded) words for the
      // residual, the input words otherwise.
      u32x4 kept_l = kept;
      if constexpr (FOLD) {
        if (lora == kLoraResidual) kept_l = kept_f;
        kept = kept_f;
      }
      __builtin_amdgcn_raw_buffer_store_b128(kept, vr, sv0, so_v, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)kcode, ir, si0, so_i, 0);
      const char* as = ring + kXStages * kXBytes + (t % kAStages) * kABytes;
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(as + c * 2048 + bo0);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(as + c * 2048 + bo1);
        const bf16x16 bf = __builtin_bit_cast(bf16x16, (u32x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
        tk[c] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, kept_l), bf, tk[c], (int)kcode, 0, 0);
        tx[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, d0), __builtin_bit_cast(bf16x8, b0), tx[c], 0, 0, 0);
        tx[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, d1), __builtin_bit_cast(bf16x8, b1), tx[c], 0, 0, 0);
      }
    }
  }
  // Drain the repeated copies before the rings become reduction arrays.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  Red& red = *reinterpret_cast<Red*>(lds);
  // Per-token L1 sums: lanes l, l^16, l^32, l^48 share a token; then across
  // wavefronts in a fixed order.
  lk += __shfl_xor(lk, 16, 64);
  lk += __shfl_xor(lk, 32, 64);
  lp += __shfl_xor(lp, 16, 64);
  lp += __shfl_xor(lp, 32, 64);
  if (lane < 16) { red.l[wave][0][lane] = lk; red.l[wave][1][lane] = lp; }
  __syncthreads();
  if (threadIdx.x < 16) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kDWaves; ++w2) { a += red.l[w2][0][threadIdx.x]; b += red.l[w2][1][threadIdx.x]; }
    // Per token, or 1 (none; per group: in the operand), or the whole
    // activation's factor, which the statistics pass left in s_out.
    const float sc = comp == kCompToken ? (a > 0.f ? (a + b) / a : 1.0f)
                   : comp == kCompTensor ? s_out[mb * 16 + threadIdx.x] : 1.0f;
    red.s[threadIdx.x] = sc;
    s_out[mb * 16 + threadIdx.x] = sc;
  }
  __syncthreads();
  // Accumulator layout of a 16x16 block: lane l holds column l % 16 of rows
  // 4 (l / 16) + i.  T_w = (X A^T)_w - c (kept A^T)_w per wavefront, then
  // summed over wavefronts in a fixed order: c = s for the residual (the
  // kept operand already folded for per-group compensation, where s = 1),
  // 1 for the pruned values, 0 for the whole input.
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * (lane >> 4) + i;
      const float cx = lora == kLoraResidual ? red.s[rr] : lora == kLoraPruned ? 1.0f : 0.0f;
      red.t[wave][rr][c * 16 + (lane & 15)] = tx[c][i] - cx * tk[c][i];
    }
  }
  __syncthreads();
  // Output fragment f = 64 rs + l: token l % 16, rank columns
  // 32 rs + 8 (l / 16) + [0, 8), four hi words then four lo words.  Thread
  // f sums its 8 columns over the wavefronts in a fixed order (two 16-byte
  // LDS reads per wavefront) and writes the fragment's hi and lo halves as
  // two 16-byte stores.
  if ((int)threadIdx.x < 64 * (int)rsteps) {
    const int rs = threadIdx.x >> 6, fl = threadIdx.x & 63, rr = fl & 15;
    const int col = 32 * rs + 8 * (fl >> 4);
    f32x4 v0 = (f32x4){0, 0, 0, 0}, v1 = (f32x4){0, 0, 0, 0};
#pragma unroll
    for (int w2 = 0; w2 < kDWaves; ++w2) {
      v0 += *reinterpret_cast<const f32x4*>(&red.t[w2][rr][col]);
      v1 += *reinterpret_cast<const f32x4*>(&red.t[w2][rr][col + 4]);
    }
    const float sr = red.s[rr];
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = alpha * v0[e] / sr; v[4 + e] = alpha * v1[e] / sr; }
    u32x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
      l[j] = pack_bf16x2(v[2 * j] - bf16_lo_to_f32(h[j]), v[2 * j + 1] - bf16_hi_to_f32(h[j]));
    }
    const int64_t o = ((mb * rsteps + rs) * 2) * 64 + fl;
    t_out[o] = h;
    t_out[o + 64] = l;
  }
}

// ---------------------------------------------------------------------------
// Per-tensor compensation: one factor for the whole activation,
// (sum of all L1) / (sum of kept L1).  Two passes before the pre-pass:
// l1_rows_kernel writes each token's kept and pruned L1 (the selection of
// the pre-pass, one wavefront per token, fixed-order lane reduction);
// tensor_scale_kernel (one workgroup) adds them in a fixed order in fp64 and
// writes the factor into every entry of the scale region, where the
// pre-pass reads it for its tokens.

template <bool A16>
__global__ void __launch_bounds__(256)
l1_rows_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, M * K * 2);
  float lk = 0.f, lp = 0.f;
  // 16 channels (4 groups) per lane and iteration, guarded by K.
  for (int64_t k = 16 * lane; k < K; k += 16 * 64) {
    uint32_t w[8];
    load_quad<A16>(xr, row, true, k, K, w);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const Group4 r = rank_group(w[2 * g], w[2 * g + 1]);
      lk = add_mag_pair(lk, r.first, r.second);
      lp = add_mag_pair(lp, r.third, r.fourth);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lk += __shfl_xor(lk, o, 64);
    lp += __shfl_xor(lp, o, 64);
  }
  if (lane == 0) {
    part[2 * row] = lk;
    part[2 * row + 1] = lp;
  }
}

__global__ void __launch_bounds__(1024)
tensor_scale_kernel(const float* __restrict__ part, int64_t M, float* __restrict__ s, int64_t mp) {
  __shared__ double red[2][1024];
  double a = 0.0, b = 0.0;
  for (int64_t i = threadIdx.x; i < M; i += 1024) {
    a += (double)part[2 * i];
    b += (double)part[2 * i + 1];
  }
  red[0][threadIdx.x] = a;
  red[1][threadIdx.x] = b;
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if ((int)threadIdx.x < h) {
      red[0][threadIdx.x] += red[0][threadIdx.x + h];
      red[1][threadIdx.x] += red[1][threadIdx.x + h];
    }
    __syncthreads();
  }
  const double lk = red[0][0], lp = red[1][0];
  const float st = lk > 0.0 ? (float)((lk + lp) / lk) : 1.0f;
  for (int64_t i = threadIdx.x; i < mp; i += 1024) s[i] = st;
}

template <bool A16>
hipError_t launch_prepass_t(const uint16_t* x, const uint16_t* lora_a, int64_t M, int64_t K,
                            int64_t r, float alpha, int comp, int lora, const WsLayout& L, char* ws,
                            hipStream_t stream) {
  // 8 workgroups per group of 8 16-token blocks, groups rounded up to a
  // multiple of 8 (the kernel's XCD-grouped mapping).
  const int64_t ngroups = L.mp / 128;
  const dim3 grid((unsigned)(64 * ((ngroups + 7) / 8))), block(64 * kWaves);
  u32x4* xv = reinterpret_cast<u32x4*>(ws + L.off_xv);
  uint16_t* xi = reinterpret_cast<uint16_t*>(ws + L.off_xi);
  float* s = reinterpret_cast<float*>(ws + L.off_s);
  u32x4* t = reinterpret_cast<u32x4*>(ws + L.off_t);
  const int64_t kpairs = L.kp / 128, rsteps = L.rp / 32;
  const int ncb = (int)(L.rp / 16);
  if (comp == kCompTensor) {
    // Per-token L1 pairs go to the operand region (2 M floats <= its
    // mp kp bytes), which the pre-pass overwrites afterwards.
    float* part = reinterpret_cast<float*>(ws + L.off_xv);
    hipError_t e = launch(&l1_rows_kernel<A16>, dim3((unsigned)((M + 3) / 4)), dim3(256), stream, x, M, K, part);
    if (e != hipSuccess) return e;
    e = launch(&tensor_scale_kernel, dim3(1), dim3(1024), stream, part, M, s, L.mp);
    if (e != hipSuccess) return e;
  }
  if constexpr (A16) {
    // r <= 64: the DMA-streamed pre-pass, one workgroup of 8 wavefronts per
    // 16-token block (same grid and mapping).
    const dim3 dblock(64 * kDWaves);
    const int64_t ksteps = L.kp / 64;
    const bool full = K % 128 == 0;
    const bool fold = comp == kCompGroup;
    if (r > 0 && ncb <= 4) {
      using Kern = decltype(&prepass_dma_kernel<2, true, true>);
      static constexpr Kern kDma[2][2][2] = {
          {{&prepass_dma_kernel<2, false, false>, &prepass_dma_kernel<2, false, true>},
           {&prepass_dma_kernel<2, true, false>, &prepass_dma_kernel<2, true, true>}},
          {{&prepass_dma_kernel<4, false, false>, &prepass_dma_kernel<4, false, true>},
           {&prepass_dma_kernel<4, true, false>, &prepass_dma_kernel<4, true, true>}}};
      return launch(kDma[ncb > 2][full][fold], grid, dblock, stream, x, lora_a, M, K, r, alpha, xv, xi, s, t,
                    ksteps, rsteps, comp, lora);
    }
  }
  const bool fold = comp == kCompGroup;
  using Kern = decltype(&prepass_kernel<A16, 0, false>);
  static constexpr Kern kGen[4][2] = {
      {&prepass_kernel<A16, 0, false>, &prepass_kernel<A16, 0, true>},
      {&prepass_kernel<A16, 2, false>, &prepass_kernel<A16, 2, true>},
      {&prepass_kernel<A16, 4, false>, &prepass_kernel<A16, 4, true>},
      {&prepass_kernel<A16, 8, false>, &prepass_kernel<A16, 8, true>}};
  const int sel = r == 0 ? 0 : ncb <= 2 ? 1 : ncb <= 4 ? 2 : 3;
  return launch(kGen[sel][fold], grid, block, stream, x, lora_a, M, K, r, alpha, xv, xi, s, t, kpairs,
                r == 0 ? (int64_t)0 : rsteps, comp, lora);
}

}  // namespace

hipError_t launch_prepass(const uint16_t* x, const uint16_t* lora_a, int64_t M, int64_t K,
                          int64_t r, float lora_scale, void* workspace, hipStream_t stream, int comp,
                          int lora) {
  const WsLayout L = ws_layout(M, K, r);
  char* ws = static_cast<char*>(workspace);
  if (K % 8 == 0) return launch_prepass_t<true>(x, lora_a, M, K, r, lora_scale, comp, lora, L, ws, stream);
  return launch_prepass_t<false>(x, lora_a, M, K, r, lora_scale, comp, lora, L, ws, stream);
}

}  // namespace rtl
