// rtl_sparsify_2of4 kernel: 2:4 pattern decision, Top-K selection, per-token
// norm-compensation scale and compression of X into the canonical
// (vals, idx) format (qingkeai RT-Lynx article, sections 01, 03.1 and 04;
// ai-feeds summary, 方法 / 核心模块 1).
//
// One or two wavefronts own one token (row).  Lanes stride over the row in
// 16-byte chunks (two groups of 4 channels), so every load instruction reads
// 1 KiB of contiguous HBM per wavefront; each chunk yields 4 kept words (8
// bytes) and one index byte.  Kept and pruned L1 mass are summed per lane in
// fp32, reduced across the wavefront with shuffles and, with two wavefronts
// per row, across the pair through LDS in a fixed order.  The kernel is bound
// by HBM: 2 bytes in, 1.125 bytes out per element.  Two wavefronts per row
// when all of them are resident at once (8 per SIMD): more loads in flight
// for the same rows (measured 16 % faster at 1152 x 3072, 8 % at
// 4096 x 12288, 2 % at 4096 x 3072; with more rows than that, one wavefront
// per row is faster: 7 % at 9216 x 3072).
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
template <bool ALIGNED16, bool FOLD, int P>
__global__ void __launch_bounds__(64 * kWaves)
sparsify_2of4_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                     uint16_t* __restrict__ vals, uint8_t* __restrict__ idx,
                     float* __restrict__ scale) {
  static_assert(P == 1 || P == 2, "one or two wavefronts per row");
  __shared__ float red[kWaves][2];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int part = wv % P;
  const int64_t row = (int64_t)blockIdx.x * (kWaves / P) + wv / P;
  if constexpr (P == 1) {
    if (row >= M) return;
  }
  const bool live = row < M;                          // both wavefronts of a row reach the barriers
  // Row sums of the P wavefronts of a row, added in wavefront order.
  auto row_sum = [&](float& a, float& b) {
    a = wave_sum(a);
    b = wave_sum(b);
    if constexpr (P > 1) {
      if (lane == 0) { red[wv][0] = a; red[wv][1] = b; }
      __syncthreads();
      const int w0 = wv - part;
      a = red[w0][0] + red[w0 + 1][0];
      b = red[w0][1] + red[w0 + 1][1];
      __syncthreads();
    }
  };
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
    for (int64_t c = part * 64 + lane; live && c < chunks; c += 64 * P) {
      uint32_t w0, w1, w2, w3;
      load_chunk(c, w0, w1, w2, w3);
      ChunkOut o;
      select_pair_groups(w0, w1, w2, w3, 2 * c + 1 < groups, o, lk, lp);
    }
    row_sum(lk, lp);
    s = lk > 0.f ? (lk + lp) / lk : 1.0f;
  }

  float lk = 0.f, lp = 0.f;
  for (int64_t c0 = 0; live && c0 < chunks; c0 += 64 * P * kUnroll) {
    uint32_t w[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + (u * P + part) * 64 + lane;
      if (c < chunks) load_chunk(c, w[u][0], w[u][1], w[u][2], w[u][3]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + (u * P + part) * 64 + lane;
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
    row_sum(lk, lp);
    if (live && part == 0 && lane == 0) scale[row] = lk > 0.f ? (lk + lp) / lk : 1.0f;
  }
}

}  // namespace

hipError_t launch_sparsify_2of4(const uint16_t* x, int64_t M, int64_t K, uint16_t* vals,
                                uint8_t* idx, float* scale, bool fold, int compute_units,
                                hipStream_t stream) {
  const bool a16 = (K % 8) == 0;
  const bool p2 = 2 * M <= 32 * (int64_t)(compute_units > 0 ? compute_units : 1);
  const int64_t rows_per = p2 ? kWaves / 2 : kWaves;
  const dim3 grid((unsigned)((M + rows_per - 1) / rows_per)), block(64 * kWaves);
  auto* k = p2 ? (a16 ? (fold ? &sparsify_2of4_kernel<true, true, 2> : &sparsify_2of4_kernel<true, false, 2>)
                      : (fold ? &sparsify_2of4_kernel<false, true, 2> : &sparsify_2of4_kernel<false, false, 2>))
               : (a16 ? (fold ? &sparsify_2of4_kernel<true, true, 1> : &sparsify_2of4_kernel<true, false, 1>)
                      : (fold ? &sparsify_2of4_kernel<false, true, 1> : &sparsify_2of4_kernel<false, false, 1>));
  return launch(k, grid, block, stream, x, M, K, vals, idx, scale);
}

}  // namespace rtl
