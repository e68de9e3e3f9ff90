// decode.hip -- expert kernels for decode and draft verification (T <= 8).
//
// Experts are multiplied straight from their low-bit blocks [strata-mlx wiki,
// opening feature list, first item]; one pass checks up to eight tokens (one
// real token and seven drafts) [devlabs blog "32GB Mac mini 6 跑 125B 大模型",
// section 核心技术特点, MTP item].
//
// Arithmetic on the matrix cores (v_mfma_f32_16x16x32_f16), transposed so the
// tokens are the M dimension and weight rows the N dimension:
//   A[m][k]  = activation fp16, m < 8: hi part of token m, m >= 8: lo part
//              of token m-8 (x = hi + lo to ~22 bits),
//   B[k][n]  = unsigned code q of weight row n, input k (exact fp16 integer),
//   C_in[m]  = -2^(b-1) * sum_k A[m][k]  (the block sum, fp32),
// so one MFMA per 32-weight block gives sum_k A (q - 2^(b-1)) = sum_k A c for
// 16 rows; the lane holding column n then applies the fp16 block scale of row
// n with one fused multiply-add per output.  Every product and the offset are
// exact; the rounding is the fp32 accumulation.
#include "kern_common.h"
#include "moe_launch.h"

namespace {

template <int BITS>
struct ChunkRegs {
  u32x4_t codes;
  u32x4_t scales;  // 8 fp16
  u32x2_t hbits;   // 3-bit only
};

template <int BITS>
DEVI void load_chunk(ChunkRegs<BITS>& c, const uint8_t* chunk, int lane) {
  c.codes = ld128_nt(chunk + 16 * lane);
  c.scales = ld128_nt(chunk + 1024 + 16 * (lane & 15));
  if constexpr (BITS == 3) c.hbits = ld64_nt(chunk + 1280 + 8 * lane);
}

template <int BITS>
DEVI half8_t chunk_frag(const ChunkRegs<BITS>& c, int f) {
  if constexpr (BITS == 2) return frag_q2(c.codes, f);
  else return frag_q3(c.codes, c.hbits, f);
}

DEVI float chunk_scale(const u32x4_t& s, int f) {
  const uint32_t dw = s[f >> 1];
  return half_bits_to_float((f & 1) ? (dw >> 16) : (dw & 0xffffu));
}

// ---------------------------------------------------------------------------
// gate/up: workgroup = (slot u, pair of 16-row tiles p) = 32 intermediate
// rows of one expert; its waves split the k-groups (256 inputs each) and
// reduce through LDS in a fixed order.  Epilogue: h = silu(g) * u, times the
// token's gate weight, written as fp16 hi/lo A-fragments of the down kernel.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(512) void gu_decode_kernel(GuArgs a) {
  constexpr int CB = BITS == 2 ? 1280 : 1792;
  __shared__ float red[8][16][64];
  __shared__ float tile[16][33];
  const int u = blockIdx.y;
  const int ns = *a.n_slots;
  if (u >= ns) return;
  const int e = a.slot_expert[u];
  const bool sh = (e == a.E);
  const int Iu = sh ? a.Is : a.I;
  const int p = blockIdx.x;
  if (32 * p >= Iu) return;
  const uint8_t* base = sh ? a.X.shared : a.X.experts + (int64_t)e * a.X.ex_stride;
  const uint8_t* gate = base + (sh ? a.X.sh_off_gate : a.X.off_gate);
  const uint8_t* up = base + (sh ? a.X.sh_off_up : a.X.off_up);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int n_kg = a.n_kg;

  float4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 2; ++r) acc[i][r] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int kg = wv; kg < n_kg; kg += nw) {
    ChunkRegs<BITS> c[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t ch = ((int64_t)(2 * p + r) * n_kg + kg) * CB;
      load_chunk<BITS>(c[0][r], gate + ch, lane);
      load_chunk<BITS>(c[1][r], up + ch, lane);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = kg * 8 + j;
      const half8_t A = *reinterpret_cast<const half8_t*>(a.xfrag + ((size_t)b * 64 + lane) * 8);
      const float4_t cin = *reinterpret_cast<const float4_t*>(a.xsum + b * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float4_t C = mfma16x16x32(A, chunk_frag<BITS>(c[mt][r], j), cin);
          const float s = chunk_scale(c[mt][r].scales, j);
          acc[mt][r] += s * C;
        }
    }
  }

  // reduce the waves' partial sums in wave order
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wv][(mt * 2 + r) * 4 + i][lane] = acc[mt][r][i];
  __syncthreads();
  if (wv == 0) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float s = red[0][q][lane];
      for (int w = 1; w < nw; ++w) s += red[w][q][lane];
      v[q] = add_partner32(s);  // hi + lo parts of the token
    }
    // lane l: column n = l & 15 (intermediate row 32p + 16r + n), rows m = 4(l>>4)+i
    const int n = lane & 15;
    const bool lo_half = lane >= 32;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 4 * ((lane >> 4) & 1) + i;
        const float g = v[(0 * 2 + r) * 4 + i];
        const float uu = v[(1 * 2 + r) * 4 + i];
        const float h = g / (1.0f + expf(-g)) * uu;
        const float gw = a.slot_w[u * 8 + tok];
        const float hs = (gw != 0.f) ? gw * h : 0.f;
        const _Float16 hi = (_Float16)hs;
        const _Float16 val = lo_half ? (_Float16)(hs - (float)hi) : hi;
        const int mrow = tok + (lo_half ? 8 : 0);
        const int kk = 16 * r + n;
        a.hfrag[(((size_t)u * a.nbI + p) * 64 + mrow + 16 * (kk >> 3)) * 8 + (kk & 7)] = val;
        tile[mrow][kk] = (float)val;
      }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float s = 0.f;
    for (int kk = 0; kk < 32; ++kk) s += tile[threadIdx.x][kk];
    a.hsum[((size_t)u * a.nbI + p) * 16 + threadIdx.x] = -(float)a.code_off * s;
  }
}

// ---------------------------------------------------------------------------
// down: workgroup = (row group rg of 16*RT output rows, split s).  It sums,
// for every slot u = s, s+S, ..., the expert's down projection of the
// gate-weighted h, so the cross-expert combine happens in the accumulators.
// Items (slot, k-group) go round-robin to the waves; waves reduce through LDS
// in a fixed order.  With S > 1 the last workgroup of a row group adds the S
// partial results in split order: the output does not depend on timing.
// ---------------------------------------------------------------------------
template <int BITS, int RT>
__global__ __launch_bounds__(512) void down_decode_kernel(DownArgs a) {
  constexpr int CB = BITS == 2 ? 1280 : 1792;
  constexpr int BK = 8 / RT;
  __shared__ float red[8][RT * 4][64];
  __shared__ int is_last;
  const int rg = blockIdx.x, sp = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int ns = *a.n_slots;

  float4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  int item = 0;
  for (int u = sp; u < ns; u += a.S) {
    const int e = a.slot_expert[u];
    const bool sh = (e == a.E);
    const int n_kg = sh ? a.n_kg_s : a.n_kg_r;
    const uint8_t* mat = sh ? a.X.shared + a.X.sh_off_down
                            : a.X.experts + (int64_t)e * a.X.ex_stride + a.X.off_down;
    for (int kg = 0; kg < n_kg; ++kg, ++item) {
      if (item % nw != wv) continue;
      ChunkRegs<BITS> c;
      load_chunk<BITS>(c, mat + ((int64_t)rg * n_kg + kg) * CB, lane);
#pragma unroll
      for (int j = 0; j < BK; ++j) {
        const int b = kg * BK + j;
        const size_t hb = (size_t)u * a.nbI + b;
        const half8_t A = *reinterpret_cast<const half8_t*>(a.hfrag + (hb * 64 + lane) * 8);
        const float4_t cin = *reinterpret_cast<const float4_t*>(a.hsum + hb * 16 + 4 * (lane >> 4));
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int f = t * BK + j;
          const float4_t C = mfma16x16x32(A, chunk_frag<BITS>(c, f), cin);
          acc[t] += chunk_scale(c.scales, f) * C;
        }
      }
    }
  }

#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][t * 4 + i][lane] = acc[t][i];
  __syncthreads();
  const int T = a.T, d = a.d;
  if (wv == 0) {
    const int n = lane & 15;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = red[0][t * 4 + i][lane];
        for (int w = 1; w < nw; ++w) s += red[w][t * 4 + i][lane];
        s = add_partner32(s);
        const int tok = 4 * (lane >> 4) + i;  // lanes < 32 hold tokens 0..7
        const int o = rg * 16 * RT + 16 * t + n;
        if (lane < 32 && tok < T) {
          if (a.S == 1) a.y[(size_t)tok * d + o] = s;
          else a.ypart[((size_t)sp * 8 + tok) * d + o] = s;
        }
      }
  }
  if (a.S == 1) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t old = atomicAdd(a.counters + rg, 1u);
    is_last = (old == (uint32_t)a.S - 1u);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const int rows = 16 * RT;
  for (int i = threadIdx.x; i < T * rows; i += blockDim.x) {
    const int tok = i / rows, o = rg * rows + (i - tok * rows);
    float s = 0.f;
    for (int q = 0; q < a.S; ++q) s += __builtin_nontemporal_load(a.ypart + ((size_t)q * 8 + tok) * d + o);
    a.y[(size_t)tok * d + o] = s;
  }
  if (threadIdx.x == 0) a.counters[rg] = 0u;
}

template <int BITS, int RT>
hipError_t launch_down_t(const DownArgs& a, int grid_x, int nw, hipStream_t s) {
  hipLaunchKernelGGL((down_decode_kernel<BITS, RT>), dim3(grid_x, a.S), dim3(64 * nw), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gu_decode(const GuArgs& a, int grid_x, int grid_y, int nw, hipStream_t s) {
  if (a.bits == 2) hipLaunchKernelGGL(gu_decode_kernel<2>, dim3(grid_x, grid_y), dim3(64 * nw), 0, s, a);
  else hipLaunchKernelGGL(gu_decode_kernel<3>, dim3(grid_x, grid_y), dim3(64 * nw), 0, s, a);
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
  }
  return hipErrorInvalidValue;
}
