// rtl_sparsify_2of4 kernel: 2:4 pattern decision, Top-K selection, per-token
// norm-compensation scale and compression of X into the canonical
// (vals, idx) format (qingkeai RT-Lynx article, sections 01, 03.1 and 04;
// ai-feeds summary, 方法 / 核心模块 1).
//
// One wavefront owns one token (row).  Lanes stride over the row in 16-byte
// chunks (two groups of 4 channels), so every load instruction reads 1 KiB of
// contiguous HBM per wavefront; each chunk yields 4 kept words (8 bytes) and
// one index byte.  Kept and pruned L1 mass are summed per lane in fp32 and
// reduced across the wavefront with DPP-free shuffles.  The kernel is bound
// by HBM: 2 bytes in, 1.125 bytes out per element.
#include "rtl_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

struct ChunkOut {
  uint32_t vals_lo, vals_hi;   // kept words of group 0 and group 1, channel order
  uint32_t code;               // group0 code | group1 code << 4
};

__device__ __forceinline__ void select_pair_groups(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                   bool has_g1, ChunkOut& o, float& lk, float& lp) {
  {
    const Group4 g = rank_group(w0, w1);
    const uint32_t sel = pair_selector_sorted(g.first, g.second);
    o.vals_lo = __builtin_amdgcn_perm(w1, w0, sel);
    o.code = code_from_selector(sel);
    lk = add_mag_pair(lk, g.first, g.second);
    lp = add_mag_pair(lp, g.third, g.fourth);
  }
  if (has_g1) {
    const Group4 g = rank_group(w2, w3);
    const uint32_t sel = pair_selector_sorted(g.first, g.second);
    o.vals_hi = __builtin_amdgcn_perm(w3, w2, sel);
    o.code |= code_from_selector(sel) << 4;
    lk = add_mag_pair(lk, g.first, g.second);
    lp = add_mag_pair(lp, g.third, g.fourth);
  } else {
    o.vals_hi = 0;
  }
}

// s * x for both words of a packed pair, rounded to bf16.
__device__ __forceinline__ uint32_t fold_pair(uint32_t w, float s) {
  return pack_bf16x2(bf16_lo_to_f32(w) * s, bf16_hi_to_f32(w) * s);
}

// ALIGNED16: K % 8 == 0, rows start on 16-byte boundaries and every chunk
// holds two whole groups.  Otherwise the row is read in 8-byte groups.
template <bool ALIGNED16, bool FOLD>
__global__ void __launch_bounds__(64 * kWaves)
sparsify_2of4_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                     uint16_t* __restrict__ vals, uint8_t* __restrict__ idx,
                     float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const int64_t groups = K / 4;
  const int64_t chunks = (groups + 1) / 2;            // = idx bytes per row
  const uint16_t* xr = x + row * K;
  uint16_t* vr = vals + row * (K / 2);
  uint8_t* ir = idx + row * chunks;

  auto load_chunk = [&](int64_t c, uint32_t& w0, uint32_t& w1, uint32_t& w2, uint32_t& w3) {
    if constexpr (ALIGNED16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c * 8);
      w0 = v[0]; w1 = v[1]; w2 = v[2]; w3 = v[3];
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2*>(xr + c * 8);
      w0 = a[0]; w1 = a[1];
      if (2 * c + 1 < groups) {
        const u32x2 b = *reinterpret_cast<const u32x2*>(xr + c * 8 + 4);
        w2 = b[0]; w3 = b[1];
      } else {
        w2 = w3 = 0;
      }
    }
  };

  float s = 1.0f;
  if constexpr (FOLD) {
    // First pass: the scale is needed before any value is written.
    float lk = 0.f, lp = 0.f;
    for (int64_t c = lane; c < chunks; c += 64) {
      uint32_t w0, w1, w2, w3;
      load_chunk(c, w0, w1, w2, w3);
      ChunkOut o;
      select_pair_groups(w0, w1, w2, w3, 2 * c + 1 < groups, o, lk, lp);
    }
    lk = wave_sum(lk);
    lp = wave_sum(lp);
    s = lk > 0.f ? (lk + lp) / lk : 1.0f;
  }

  float lk = 0.f, lp = 0.f;
  for (int64_t c0 = 0; c0 < chunks; c0 += 64 * kUnroll) {
    uint32_t w[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * 64 + lane;
      if (c < chunks) load_chunk(c, w[u][0], w[u][1], w[u][2], w[u][3]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * 64 + lane;
      if (c < chunks) {
        const bool has_g1 = 2 * c + 1 < groups;
        ChunkOut o;
        select_pair_groups(w[u][0], w[u][1], w[u][2], w[u][3], has_g1, o, lk, lp);
        if constexpr (FOLD) {
          o.vals_lo = fold_pair(o.vals_lo, s);
          o.vals_hi = fold_pair(o.vals_hi, s);
        }
        if constexpr (ALIGNED16) {
          *reinterpret_cast<u32x2*>(vr + c * 4) = (u32x2){o.vals_lo, o.vals_hi};
        } else {
          *reinterpret_cast<uint32_t*>(vr + c * 4) = o.vals_lo;
          if (has_g1) *reinterpret_cast<uint32_t*>(vr + c * 4 + 2) = o.vals_hi;
        }
        ir[c] = (uint8_t)o.code;
      }
    }
  }
  if (scale != nullptr) {
    lk = wave_sum(lk);
    lp = wave_sum(lp);
    if (lane == 0) scale[row] = lk > 0.f ? (lk + lp) / lk : 1.0f;
  }
}

}  // namespace

hipError_t launch_sparsify_2of4(const uint16_t* x, int64_t M, int64_t K, uint16_t* vals,
                                uint8_t* idx, float* scale, bool fold, hipStream_t stream) {
  const dim3 grid((unsigned)((M + kWaves - 1) / kWaves)), block(64 * kWaves);
  const bool a16 = (K % 8) == 0;
  auto* k = a16 ? (fold ? &sparsify_2of4_kernel<true, true> : &sparsify_2of4_kernel<true, false>)
                 : (fold ? &sparsify_2of4_kernel<false, true> : &sparsify_2of4_kernel<false, false>);
  return launch(k, grid, block, stream, x, M, K, vals, idx, scale);
}

}  // namespace rtl
