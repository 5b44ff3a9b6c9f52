// Canonical compressed activation -> the structured-sparse GEMM's operand
// order (rtl_sparse_linear_compressed).
//
// Input: the format rtl_sparsify_2of4 writes (the compression step of the
// qingkeai RT-Lynx article, section 04): vals [M, K/2] bf16, the kept pair of
// group g at columns 2g, 2g + 1; idx [M, ceil(K/8)] bytes, group g's code
// idx0 | idx1 << 2 in byte g / 2 (low nibble for even g); scale [M] fp32 or
// none (s = 1).  Output: the workspace regions the pre-pass fills (compressed
// operand words, position fields, per-token scale), so that the GEMM of
// rtl_sparse_linear_apply runs on them unchanged with r = 0.
//
// Both formats list a row's kept values in channel order, so a lane's 8
// operand words of a k-step (groups 4q .. 4q + 3 of its token, q = lane / 16)
// are 16 consecutive bytes of the canonical row, and its 16-bit position
// field is the little-endian pair of bytes 8 ks + 2q, 8 ks + 2q + 1 of the
// index row (group 4q in the lowest nibble, as the pre-pass builds it).
// Channels past K (the workspace pads K to 128) become zero words with the
// code of an all-zero group (positions 0, 1), tokens past M zero words.
//
// Grid: one workgroup of 512 threads per (8-block group, k-step); thread
// (block sub, lane) writes one 16-byte operand chunk and one field.  Pure
// data movement: HBM-bound, 2 x 1.125 M K bytes.
#include "rtl_common.hpp"
#include "rtl_kernels.hpp"

namespace rtl {

namespace {

template <bool ALIGNED16>
__global__ void __launch_bounds__(512)
repack_kernel(const uint16_t* __restrict__ vals, const uint8_t* __restrict__ idx,
              const float* __restrict__ scale, int64_t M, int64_t K, u32x4* __restrict__ xv,
              uint16_t* __restrict__ xi, float* __restrict__ s_out, int64_t ksteps) {
  const int lane = threadIdx.x & 63, sub = threadIdx.x >> 6;
  const int64_t grp = blockIdx.x / ksteps, ks = blockIdx.x % ksteps;
  const int q = lane >> 4;
  const int64_t row = (grp * 8 + sub) * 16 + (lane & 15);
  const int64_t half = K / 2;                       // compressed values per row
  const int64_t nb = (K / 4 + 1) / 2;               // index bytes per row
  const int64_t v0 = ks * 32 + 8 * q;               // first compressed value of the lane
  const bool row_ok = row < M;

  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vals, M * half * 2);
  u32x4 w = (u32x4){0, 0, 0, 0};
  if constexpr (ALIGNED16) {
    // K % 16 == 0: a lane's 16 bytes lie inside the row or wholly past K.
    const bool ok = row_ok && v0 + 8 <= half;
    w = buf_load16(vr, ok ? (uint32_t)((row * half + v0) * 2) : kOobOffset);
  } else {
    // K % 4 == 0 only: pairs of values (one group each) never straddle K.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = row_ok && v0 + 2 * j + 2 <= half;
      w[j] = __builtin_amdgcn_raw_buffer_load_b32(vr, ok ? (uint32_t)((row * half + v0 + 2 * j) * 2) : kOobOffset, 0, 0);
    }
  }

  // Position field: 4 codes, group 4q + e in nibble e.  Groups past K/4
  // (and tokens past M) get code 4 (positions 0, 1) over zero words.
  const __amdgpu_buffer_rsrc_t ir = make_rsrc(idx, M * nb);
  uint32_t field = 0;
  const int64_t g0 = ks * 16 + 4 * q;               // first group of the lane
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    const int64_t byte = (g0 + e) / 2;              // holds groups g0 + e, g0 + e + 1
    const bool ok = row_ok && byte < nb;
    const uint32_t b = ok ? __builtin_amdgcn_raw_buffer_load_b8(ir, (uint32_t)(row * nb + byte), 0, 0) : 0u;
    uint32_t lo = b & 0xfu, hi = b >> 4;
    if (!(row_ok && g0 + e < K / 4)) lo = 4u;
    if (!(row_ok && g0 + e + 1 < K / 4)) hi = 4u;
    field |= (lo | (hi << 4)) << (4 * e);
  }

  xv[((grp * ksteps + ks) * 8 + sub) * 64 + lane] = w;
  xi[((grp * ksteps + ks) * 64 + lane) * 8 + sub] = (uint16_t)field;
  if (ks == 0 && q == 0) s_out[row] = (scale != nullptr && row_ok) ? scale[row] : 1.0f;
}

}  // namespace

hipError_t launch_repack(const uint16_t* vals, const uint8_t* idx, const float* scale, int64_t M,
                         int64_t K, void* workspace, hipStream_t stream) {
  const WsLayout L = ws_layout(M, K, 0);
  char* ws = static_cast<char*>(workspace);
  u32x4* xv = reinterpret_cast<u32x4*>(ws + L.off_xv);
  uint16_t* xi = reinterpret_cast<uint16_t*>(ws + L.off_xi);
  float* s = reinterpret_cast<float*>(ws + L.off_s);
  const int64_t ngroups = L.mp / 128, ksteps = L.kp / 64;
  const dim3 grid((unsigned)(ngroups * ksteps)), block(512);
  auto* k = K % 16 == 0 ? &repack_kernel<true> : &repack_kernel<false>;
  return launch(k, grid, block, stream, vals, idx, scale, M, K, xv, xi, s, ksteps);
}

}  // namespace rtl
