// pack.hip -- re-tile canonical low-bit blocks into the lane-chunked layout
// the expert kernels stream (integer shuffling only: codes stay b-bit and
// scales stay fp16), and the test-only export that decodes weights back out of
// that layout.
//
// Canonical block (input): fp16 scale (little endian) then 4b code bytes;
// code j = bits [b*j, b*j+b) of the code bytes' little-endian bitstream,
// value q_j - 2^(b-1).  Codebook blocks (kind MOE_KIND_CB, 15 bytes): fp16
// scale, the low bytes of eight 9-bit grid indices (index i: inputs
// 4i..4i+3), a byte of index high bits (bit i), then 32 sign bits (bit j of
// the little-endian word: input j negative); the packed chunk keeps the same
// fields, regrouped per lane.  Keeping experts in their low-bit blocks and
// multiplying from them is the method of the strata-mlx wiki (opening
// feature list, first item); the block structure follows the ggml block types
// named in that wiki's credits list.
#include "kern_common.h"
#include "moe_launch.h"

namespace {

struct PackArgs {
  const uint8_t* canon;        // matrix of expert 0 in the canonical buffer
  int64_t canon_stride;        // bytes between consecutive experts (canonical)
  uint8_t* out;                // matrix of expert 0 in the packed buffer
  int64_t out_stride;          // bytes between consecutive experts (packed)
  int32_t n_experts, cols, bits, BK, RT, n_rg, n_kg, chunk_bytes;
  uint32_t* bad_scale;         // set to 1 if any scale is inf/nan or |s| >= 8192
};

__global__ __launch_bounds__(256) void pack_matrix_kernel(PackArgs a) {
  const int64_t per_expert = (int64_t)a.n_rg * a.n_kg * 64;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= per_expert * a.n_experts) return;
  const int e = (int)(gid / per_expert);
  const int64_t r = gid - (int64_t)e * per_expert;
  const int lane = (int)(r & 63);
  const int64_t chunk = r >> 6;
  const int rg = (int)(chunk / a.n_kg), kg = (int)(chunk - (int64_t)rg * a.n_kg);
  const int n = lane & 15, q = lane >> 4;
  const bool cbk = a.bits == MOE_KIND_CB;
  const int bb = cbk ? 15 : 2 + 4 * a.bits, nb = a.cols / 32;
  const uint8_t* cb = a.canon + (int64_t)e * a.canon_stride;
  uint8_t* ob = a.out + (int64_t)e * a.out_stride + chunk * a.chunk_bytes;

  uint32_t dw[4] = {0u, 0u, 0u, 0u};
  uint32_t hw[2] = {0u, 0u};
  uint32_t sc[4] = {0u, 0u, 0u, 0u};
  uint32_t ih = 0u;
  bool bad = false;
  for (int f = 0; f < 8; ++f) {
    const int t = f / a.BK, j = f - t * a.BK;
    const int64_t row = (int64_t)rg * 16 * a.RT + 16 * t + n;
    const int blk = kg * a.BK + j;
    const uint8_t* B = cb + (row * nb + blk) * bb;
    const uint32_t s = (uint32_t)B[0] | ((uint32_t)B[1] << 8);
    // b-bit codes: exponent field 28..31 (|s| >= 8192, inf or nan); codebook
    // magnitudes reach 127, so there |s| >= 256 (0x5C00) is refused: s * c
    // then stays below 2^15 in fp16, as for the b-bit codes
    bad |= (s & 0x7fffu) >= (cbk ? 0x5C00u : 0x7000u);
    sc[f >> 1] |= s << (16 * (f & 1));
    if (cbk) {
      // indices 2q, 2q+1 (inputs 8q..8q+7), their high bits, sign byte q
      dw[f >> 1] |= ((uint32_t)B[2 + 2 * q] | ((uint32_t)B[3 + 2 * q] << 8)) << (16 * (f & 1));
      ih |= ((uint32_t)(B[10] >> (2 * q)) & 3u) << (2 * f);
      hw[f >> 2] |= (uint32_t)B[11 + q] << (8 * (f & 3));
      continue;
    }
    uint32_t v;
    if (a.bits == 2) {
      v = (uint32_t)B[2 + 2 * q] | ((uint32_t)B[3 + 2 * q] << 8);
    } else {
      v = (uint32_t)B[2 + 3 * q] | ((uint32_t)B[3 + 3 * q] << 8) | ((uint32_t)B[4 + 3 * q] << 16);
    }
    for (int c = 0; c < 8; ++c) {
      const uint32_t qv = (v >> (a.bits * c)) & ((1u << a.bits) - 1u);
      dw[f >> 1] |= (qv & 3u) << (4 * c + 2 * (f & 1));
      if (a.bits == 3) hw[f >> 2] |= (qv >> 2) << (4 * c + (f & 3));
    }
  }
  *reinterpret_cast<u32x4_t*>(ob + 16 * lane) = u32x4_t{dw[0], dw[1], dw[2], dw[3]};
  if (q == 0) *reinterpret_cast<u32x4_t*>(ob + 1024 + 16 * n) = u32x4_t{sc[0], sc[1], sc[2], sc[3]};
  if (a.bits != 2) *reinterpret_cast<u32x2_t*>(ob + 1280 + 8 * lane) = u32x2_t{hw[0], hw[1]};
  if (cbk) *reinterpret_cast<uint16_t*>(ob + 1792 + 2 * lane) = (uint16_t)ih;
  if (bad) atomicOr(a.bad_scale, 1u);
}

// The codebook grid of a layer: 512 x 4 unsigned magnitudes (bytes) to fp16
// (exact), rejecting magnitudes above 127 through the status word.
__global__ __launch_bounds__(256) void pack_grid_kernel(const uint8_t* grid, uint16_t* out, uint32_t* bad) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= 512 * 4) return;
  const uint32_t m = grid[i];
  const _Float16 h = (_Float16)(float)m;
  uint16_t hb;
  __builtin_memcpy(&hb, &h, 2);
  out[i] = hb;
  if (m > 127u) atomicOr(bad, 2u);
}

struct UnpackArgs {
  const uint8_t* mat;  // packed matrix
  const uint16_t* grid16;  // codebook blocks: fp16 grid [512][4]
  int32_t rows, cols, bits, BK, RT, n_kg, chunk_bytes;
  int8_t* codes;
  float* w32;
  uint16_t* w16;
};

__global__ __launch_bounds__(256) void debug_unpack_kernel(UnpackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.rows * a.cols) return;
  const int row = (int)(gid / a.cols), col = (int)(gid - (int64_t)row * a.cols);
  const int blk = col >> 5, k = col & 31, q = k >> 3, c = k & 7;
  const int rows_rg = 16 * a.RT;
  const int rg = row / rows_rg, t = (row - rg * rows_rg) >> 4, n = row & 15;
  const int kg = blk / a.BK, j = blk - kg * a.BK, f = t * a.BK + j;
  const int lane = n + 16 * q;
  const uint8_t* ch = a.mat + ((int64_t)rg * a.n_kg + kg) * a.chunk_bytes;
  int code;
  if (a.bits == MOE_KIND_CB) {
    const int i = c >> 2;  // first or second index of the fragment
    const uint32_t lo = ch[16 * lane + 2 * f + i];
    const uint32_t hb = *reinterpret_cast<const uint16_t*>(ch + 1792 + 2 * lane);
    const uint32_t index = lo | (((hb >> (2 * f + i)) & 1u) << 8);
    const int m = (int)half_bits_to_float(a.grid16[4 * index + (c & 3)]);
    const uint32_t sg = ch[1280 + 8 * lane + f];
    code = ((sg >> c) & 1u) ? -m : m;
  } else {
    const uint32_t dw = *reinterpret_cast<const uint32_t*>(ch + 16 * lane + 4 * (f >> 1));
    uint32_t qv = (dw >> (4 * c + 2 * (f & 1))) & 3u;
    if (a.bits == 3) {
      const uint32_t hw = *reinterpret_cast<const uint32_t*>(ch + 1280 + 8 * lane + 4 * (f >> 2));
      qv += 4u * ((hw >> (4 * c + (f & 3))) & 1u);
    }
    code = (int)qv - (1 << (a.bits - 1));
  }
  const uint32_t sb = *reinterpret_cast<const uint16_t*>(ch + 1024 + 16 * n + 2 * f);
  const float w = half_bits_to_float(sb) * (float)code;  // exact: <= 18 significant bits
  if (a.codes) a.codes[gid] = (int8_t)code;
  if (a.w32) a.w32[gid] = w;
  if (a.w16) {
    _Float16 h = (_Float16)w;  // round to nearest even
    uint16_t hb;
    __builtin_memcpy(&hb, &h, 2);
    a.w16[gid] = hb;
  }
}

}  // namespace

hipError_t launch_pack_matrix(const uint8_t* canon, int64_t canon_stride, uint8_t* out, int64_t out_stride,
                              int n_experts, const moe_mat_layout& L, int bits, uint32_t* bad_scale,
                              hipStream_t s) {
  PackArgs a{canon, canon_stride, out, out_stride, n_experts, L.cols, bits, L.BK, L.RT, L.n_rg, L.n_kg,
             L.chunk_bytes, bad_scale};
  const int64_t threads = (int64_t)L.n_rg * L.n_kg * 64 * n_experts;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_matrix_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_grid(const uint8_t* grid, uint16_t* out, uint32_t* bad, hipStream_t s) {
  hipLaunchKernelGGL(pack_grid_kernel, dim3(8), dim3(256), 0, s, grid, out, bad);
  return hipGetLastError();
}

hipError_t launch_debug_unpack(const uint8_t* mat, const uint16_t* grid16, const moe_mat_layout& L, int bits,
                               int8_t* codes, float* w32, uint16_t* w16, hipStream_t s) {
  UnpackArgs a{mat, grid16, L.rows, L.cols, bits, L.BK, L.RT, L.n_kg, L.chunk_bytes, codes, w32, w16};
  const int64_t n = (int64_t)L.rows * L.cols;
  const int64_t blocks = (n + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}
