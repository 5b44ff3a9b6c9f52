// Shared device-side helpers of librtlynx (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace rtl {

// Host-side launch of kernel k that returns this launch's own status
// (hipLaunchKernel), instead of reading the thread's last-error slot after a
// triple-chevron launch: an earlier asynchronous error of the caller is then
// neither reported as the library's failure nor cleared.  The arguments are
// converted to the kernel's parameter types first.
template <typename Kern, typename Tuple, size_t... I>
inline hipError_t launch_tuple(Kern k, dim3 grid, dim3 block, hipStream_t stream, Tuple& t,
                               std::index_sequence<I...>) {
  void* ptrs[] = {static_cast<void*>(&std::get<I>(t))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, stream);
}

template <typename... P, typename... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t stream, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<std::decay_t<P>...> args(std::forward<A>(a)...);
  return launch_tuple(k, grid, block, stream, args, std::index_sequence_for<P...>{});
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Workspace layout of the fused sparse-linear path.  Rows are padded to a
// multiple of 256 (one GEMM tile), K to a multiple of 128 (two 64-deep
// structured-sparse k-steps share one 32-bit index word), the LoRA rank to a
// multiple of 32 (one dense 16x16x32 k-step).
//
//   xv: compressed values, 16-token blocks mb grouped in eights:
//       [mb / 8][k-step][mb % 8][lane] x 16 bytes, so the 8 fragments one
//       wavefront needs for a k-step are 8 KiB contiguous;
//   xi: 2-bit positions, 16 bits per lane and k-step (the lane's four
//       groups), [mb / 8][k-step][lane][mb % 8] x 2 bytes, so one 16-byte
//       read gives a lane the fields of all 8 row blocks;
//   s:  per-token scale, fp32 [mp];
//   t:  alpha * T / s as bf16 hi and lo, [mb][r-step][hi, lo][lane] x 16 bytes.
// ---------------------------------------------------------------------------
struct WsLayout {
  int64_t mp, kp, rp;
  size_t off_xv, off_xi, off_s, off_t, total;
};

__host__ __device__ inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

__host__ __device__ inline WsLayout ws_layout(int64_t M, int64_t K, int64_t r) {
  WsLayout L;
  L.mp = round_up(M, 256);
  L.kp = round_up(K, 128);
  L.rp = round_up(r, 32);
  size_t o = 0;
  L.off_xv = o; o += (size_t)L.mp * (size_t)L.kp;                 // (mp/16)(kp/64) x 1 KiB
  o = (size_t)round_up((int64_t)o, 256);
  L.off_xi = o; o += (size_t)L.mp * (size_t)L.kp / 8;             // (mp/128)(kp/64) x 64 lanes x 8 x 2 B
  o = (size_t)round_up((int64_t)o, 256);
  L.off_s = o; o += (size_t)L.mp * 4;
  o = (size_t)round_up((int64_t)o, 256);
  L.off_t = o; o += (size_t)L.mp * (size_t)L.rp * 4;              // hi and lo bf16 per element
  o = (size_t)round_up((int64_t)o, 256);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// Top-2-of-4 selection on one group of 4 bf16 words.
//
// lo = x1:x0 and hi = x3:x2 (x0 in the low half).  Each element gets a
// 32-bit composite key: its 15-bit magnitude (the bf16 word without its sign
// bit) in bits 30..16, which orders like |x| for every finite value and ties
// -0 with +0, and a position code 0x0202*(3-i) in bits 15..0.  The position
// code makes every key distinct and ranks the lower index higher among equal
// magnitudes, so the two largest composites are exactly the kept pair with
// ties resolved toward the lower channel.  The position code of element i is
// also 0x0706 - (byte selector of x_i inside hi:lo), which turns a key
// straight into a v_perm_b32 selector.
//
// Because the magnitude sits in the upper 16 bits with the low 16 cleared,
// (key & 0xffff0000) is |x_i| as an fp32 bit pattern.
// ---------------------------------------------------------------------------
struct Group4 {
  uint32_t first, second, third, fourth;   // composite keys, descending
};

__device__ __forceinline__ Group4 rank_group(uint32_t lo, uint32_t hi) {
  const uint32_t c0 = ((lo << 16) & 0x7fff0000u) | 0x0606u;
  const uint32_t c1 = (lo & 0x7fff0000u) | 0x0404u;
  const uint32_t c2 = ((hi << 16) & 0x7fff0000u) | 0x0202u;
  const uint32_t c3 = hi & 0x7fff0000u;
  const uint32_t t = max(max(c0, c1), c2);                  // v_max3_u32
  const uint32_t u = max(min(c0, c1), min(max(c0, c1), c2)); // median, v_med3_u32
  const uint32_t v = min(min(c0, c1), c2);                  // v_min3_u32
  Group4 g;
  g.first = max(t, c3);
  g.second = max(u, min(t, c3));
  g.third = max(v, min(u, c3));
  g.fourth = min(v, c3);
  return g;
}

// v_perm_b32 selector that packs the words named by keys a and b as
// (word_lower_index) | (word_higher_index) << 16, i.e. in channel order.
__device__ __forceinline__ uint32_t pair_selector_sorted(uint32_t ka, uint32_t kb) {
  const uint32_t pa = ka & 0xffffu, pb = kb & 0xffffu;   // larger code = lower index
  const uint32_t hi_code = max(pa, pb), lo_code = min(pa, pb);
  return 0x07060706u - (hi_code | (lo_code << 16));
}

// In-group positions (0..3) from a sorted selector: byte 0 = 2*idx0, byte 2 = 2*idx1.
__device__ __forceinline__ uint32_t code_from_selector(uint32_t sel) {
  return ((sel >> 1) & 3u) | ((sel >> 15) & 0xcu);        // idx0 | idx1 << 2
}

// |a| + |b| of the two magnitudes held in the upper halves of keys ka, kb,
// added to acc in fp32 (bf16 dot product against (1, 1)).
__device__ __forceinline__ float add_mag_pair(float acc, uint32_t ka, uint32_t kb) {
  const uint32_t packed = __builtin_amdgcn_perm(kb, ka, 0x07060302u);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// fp32 -> bf16 round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
}

// The same rounding of two values by the hardware's packed conversion
// (v_cvt_pk_bf16_f32, round to nearest even): a in the low half, b in the
// high half.  One instruction instead of two per value; the GEMM epilogues
// convert every output with it.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Variants of the layer that the pages leave open (rtl_sparse_linear_prepare_variant).
// Compensation: per token (default), none, one factor for the whole
// activation, or per group of 4 folded into the kept values.
constexpr int kCompToken = 0, kCompNone = 1, kCompTensor = 2, kCompGroup = 3;
// LoRA input: the pruned residual X - S(X) (default), the pruned values
// (1 - M) * X, or the whole input X.
constexpr int kLoraResidual = 0, kLoraPruned = 1, kLoraInput = 2;

// fp64 -> bf16, round to nearest even (finite inputs; values past the bf16
// range give infinity).  Normal results round the fp64 significand at its
// bit 45; results below 2^-126 are multiples of 2^-133, the bf16 subnormal
// quantum.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double q) {
  const uint64_t u = __builtin_bit_cast(uint64_t, q);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const double a = __builtin_fabs(q);
  if (a < 0x1p-126) return sign | (uint32_t)__builtin_rint(a * 0x1p133);
  uint64_t b = u & 0x7fffffffffffffffull;
  b += 0x00000fffffffffffull + ((b >> 45) & 1u);
  const int64_t e = (int64_t)(b >> 52) - 1023;
  if (e > 127) return sign | 0x7f80u;
  return sign | ((uint32_t)(e + 127) << 7) | ((uint32_t)(b >> 45) & 0x7fu);
}

// The kept pair of one group (operand word, channel order) scaled by the
// group's compensation factor -- L1 of the group over L1 of the kept pair --
// and rounded to bf16 once: each value is formed as
// (x * L1 group) / L1 kept in fp64, from the exact magnitudes, so the
// product and the sums are exact (for magnitudes within 2^45 of each other,
// i.e. any group but pathological ones) and the one correctly rounded
// division makes the bf16 rounding that of the exact value.  A zero kept
// pair (a zero group) is returned as it is.
__device__ __forceinline__ uint32_t fold_group(uint32_t kept_word, const Group4& g) {
  const double a = (double)__builtin_bit_cast(float, g.first & 0xffff0000u);
  const double b = (double)__builtin_bit_cast(float, g.second & 0xffff0000u);
  const double c = (double)__builtin_bit_cast(float, g.third & 0xffff0000u);
  const double d = (double)__builtin_bit_cast(float, g.fourth & 0xffff0000u);
  const double lk = a + b;
  if (!(lk > 0.0)) return kept_word;
  const double tot = lk + c + d;
  const double v0 = (double)bf16_lo_to_f32(kept_word), v1 = (double)bf16_hi_to_f32(kept_word);
  return f64_to_bf16_rne(v0 * tot / lk) | (f64_to_bf16_rne(v1 * tot / lk) << 16);
}

// Buffer resource over a whole tensor (raw, stride 0): loads past `bytes`
// return zeros instead of faulting, stores there are dropped.  The host
// keeps every tensor below 2 GiB, so sizes and offsets fit 32 bits.  Guarded
// loads through it need no branch: an out-of-range element gets an offset
// past the end (kOobOffset) and reads as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Byte offset that lies past every tensor: a buffer load there returns zeros.
constexpr uint32_t kOobOffset = 0xfffffff0u;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}

}  // namespace rtl
