// decode.hip -- the decode path as three kernels per layer (route.hip's
// router, then gate/up and down here), for stacks whose layers differ in
// shape; the persistent stack kernel (persist.hip) runs the same device code
// (decode_dev.h) as phases of one launch.
#include "decode_dev.h"

namespace {

// gate/up: one workgroup of 8 wavefronts per CU (the grid is the CU count);
// every workgroup selects the experts of every token itself and builds the
// slot list, workgroup 0 publishes the routing and the slot list.
template <int BITS, int NPER, int AM>
__global__ __launch_bounds__(64 * GU_NW) void gu_decode_kernel(GuArgs a) {
  __shared__ GuLds L;
  load_grid<BITS>(a.X.grid16, threadIdx.x, 64 * GU_NW);  // (the selection's barriers publish it)
  // the first sh_wgs workgroups run the shared expert's items (they do not
  // depend on the routing, so no selection delays them); the others select
  // and run the routed experts' items (with sh_wgs = 0, every workgroup
  // selects and runs its share of all items)
  const int nsh = a.sh_wgs;
  if ((int)blockIdx.x < nsh) {
    gu_prologue_shared<AM>(a, L);
    gu_items<BITS, AM>(a, L, blockIdx.x, nsh, nullptr, 1);
  } else {
    const bool first = (int)blockIdx.x == nsh;
    gu_select<BITS, NPER, AM>(a, L, first, first);
    gu_items<BITS, AM>(a, L, blockIdx.x - nsh, gridDim.x - nsh, nullptr, nsh > 0 ? 2 : 0);
  }
}

// down: workgroup = (row group, split), the slot list from the workspace.
template <int BITS, int RT, int AM>
__global__ __launch_bounds__(512) void down_decode_kernel(DownArgs a) {
  __shared__ float red[8 * RT * 4 * 64];
  if constexpr (BITS == MOE_KIND_CB) {
    load_grid<BITS>(a.X.grid16, threadIdx.x, blockDim.x);
    __syncthreads();
  }
  down_role<BITS, RT, AM>(a, blockIdx.x, blockIdx.y, *a.n_slots, a.slot_expert, red);
}

// ---------------------------------------------------------------------------
// Test export of one packed matrix through this file's own decoders: one
// wavefront per chunk loads it with load_chunk and, for each of its 8
// fragments, takes the codes from chunk_frag (the matrix-core B operand:
// unsigned for b-bit blocks, signed for codebook blocks) and the block scale
// from chunk_scale (the epilogue factor).  Lane l = n + 16 q writes row
// 16 (RT rg + t) + n, inputs 32 (BK kg + j) + 8 q + c of fragment f = BK t + j:
// the signed code (q_c - 2^(b-1), or the codebook's) and scale times code
// (exact in fp32).
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void debug_decode_path_kernel(DebugPathArgs a) {
  const int chunk = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if constexpr (BITS == MOE_KIND_CB) {
    load_grid<BITS>(a.grid16, threadIdx.x, blockDim.x);
    __syncthreads();
  }
  if (chunk >= a.n_rg * a.n_kg) return;
  const int rg = chunk / a.n_kg, kg = chunk - rg * a.n_kg;
  const int n = lane & 15, q = lane >> 4;
  ChunkRegs<BITS> c;
  load_chunk<BITS>(c, a.mat + (int64_t)chunk * a.chunk_bytes, lane);
  const int off = moe_code_offset(BITS);
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int t = f / a.BK, j = f - t * a.BK;
    const int row = (rg * a.RT + t) * 16 + n;
    const int col = 32 * (kg * a.BK + j) + 8 * q;
    const half8_t qv = chunk_frag<BITS>(c, f);
    const float s = chunk_scale(c.scales, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int code = (int)(float)qv[e] - off;
      const size_t o = (size_t)row * a.cols + col + e;
      if (a.codes) a.codes[o] = (int8_t)code;
      if (a.w32) a.w32[o] = s * (float)code;
    }
  }
}

template <int BITS, int RT>
hipError_t launch_down_t(const DownArgs& a, int grid_x, int nw, hipStream_t s) {
  if (a.am == MOE_AM_HL16) MOE_LAUNCH((down_decode_kernel<BITS, RT, MOE_AM_HL16>), dim3(grid_x, a.S), dim3(64 * nw), 0, s, a);
  else if (a.am == MOE_AM_F16) MOE_LAUNCH((down_decode_kernel<BITS, RT, MOE_AM_F16>), dim3(grid_x, a.S), dim3(64 * nw), 0, s, a);
  else MOE_LAUNCH((down_decode_kernel<BITS, RT, MOE_AM_HL8>), dim3(grid_x, a.S), dim3(64 * nw), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gu_decode(const GuArgs& a, int n_wg, hipStream_t s) {
#define GU_LAUNCH(B, N)                                                                     \
  do {                                                                                      \
    if (a.am == MOE_AM_HL16) MOE_LAUNCH((gu_decode_kernel<B, N, MOE_AM_HL16>), dim3(n_wg), dim3(64 * GU_NW), 0, s, a); \
    else if (a.am == MOE_AM_F16) MOE_LAUNCH((gu_decode_kernel<B, N, MOE_AM_F16>), dim3(n_wg), dim3(64 * GU_NW), 0, s, a); \
    else MOE_LAUNCH((gu_decode_kernel<B, N, MOE_AM_HL8>), dim3(n_wg), dim3(64 * GU_NW), 0, s, a);                      \
  } while (0)
  const int np = a.E <= 512 ? 8 : a.E <= 1024 ? 16 : a.E <= 2048 ? 32 : 64;
  if (a.bits == 2) {
    if (np == 8) GU_LAUNCH(2, 8);
    else if (np == 16) GU_LAUNCH(2, 16);
    else if (np == 32) GU_LAUNCH(2, 32);
    else GU_LAUNCH(2, 64);
  } else if (a.bits == MOE_KIND_CB) {
    if (np == 8) GU_LAUNCH(MOE_KIND_CB, 8);
    else if (np == 16) GU_LAUNCH(MOE_KIND_CB, 16);
    else if (np == 32) GU_LAUNCH(MOE_KIND_CB, 32);
    else GU_LAUNCH(MOE_KIND_CB, 64);
  } else {
    if (np == 8) GU_LAUNCH(3, 8);
    else if (np == 16) GU_LAUNCH(3, 16);
    else if (np == 32) GU_LAUNCH(3, 32);
    else GU_LAUNCH(3, 64);
  }
#undef GU_LAUNCH
  return hipGetLastError();
}

hipError_t launch_debug_decode_path(const DebugPathArgs& a, int bits, hipStream_t s) {
  const int n = a.n_rg * a.n_kg;
  if (n == 0) return hipSuccess;
  if (bits == 2) hipLaunchKernelGGL(debug_decode_path_kernel<2>, dim3((n + 3) / 4), dim3(256), 0, s, a);
  else if (bits == 3) hipLaunchKernelGGL(debug_decode_path_kernel<3>, dim3((n + 3) / 4), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(debug_decode_path_kernel<MOE_KIND_CB>, dim3((n + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_decode(const DownArgs& a, int grid_x, int nw, hipStream_t s) {
  switch (a.RT * 10 + a.bits) {
    case 12: return launch_down_t<2, 1>(a, grid_x, nw, s);
    case 22: return launch_down_t<2, 2>(a, grid_x, nw, s);
    case 42: return launch_down_t<2, 4>(a, grid_x, nw, s);
    case 82: return launch_down_t<2, 8>(a, grid_x, nw, s);
    case 13: return launch_down_t<3, 1>(a, grid_x, nw, s);
    case 23: return launch_down_t<3, 2>(a, grid_x, nw, s);
    case 43: return launch_down_t<3, 4>(a, grid_x, nw, s);
    case 83: return launch_down_t<3, 8>(a, grid_x, nw, s);
    case 10 + MOE_KIND_CB: return launch_down_t<MOE_KIND_CB, 1>(a, grid_x, nw, s);
    case 20 + MOE_KIND_CB: return launch_down_t<MOE_KIND_CB, 2>(a, grid_x, nw, s);
    case 40 + MOE_KIND_CB: return launch_down_t<MOE_KIND_CB, 4>(a, grid_x, nw, s);
    case 80 + MOE_KIND_CB: return launch_down_t<MOE_KIND_CB, 8>(a, grid_x, nw, s);
  }
  return hipErrorInvalidValue;
}
