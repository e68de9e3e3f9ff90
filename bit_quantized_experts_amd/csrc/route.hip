// route.hip -- router GEMV, top-k selection with gate weights, the expert
// slot list for the decode kernels, RMSNorm between stacked layers.
//
// The router keeps about ten of 512 small experts per token [cnyes profile of
// Strata, section "Strata 到底是什麼？"]; it stays resident next to the
// shared expert [same page, section "三層記憶體", part 1].
//
// Decode (T <= 8) splits the router GEMV over column slices of the input so
// that no workgroup needs the whole input row: the previous layer's output
// arrives as split partial sums, and each workgroup adds only the 256 columns
// it multiplies.  RMSNorm is a per-token scale, so it is applied after the
// dot products (logit = (y . w) / rms(y) + bias) and, in the expert kernels,
// to the accumulators before the SwiGLU nonlinearity.
#include "kern_common.h"
#include "moe_launch.h"

namespace {

// Selection key of (logit v, expert e): larger key = ranks earlier (logit
// descending, then index ascending).  The float's bits are mapped to an
// unsigned integer of the same order (-0.0 first folded into +0.0); the low
// word is the complement of the index.  Key 0 never occurs for a finite
// logit, so it marks an expert already taken.
DEVI uint64_t sel_key(float v, int e) {
  uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
DEVI float key_value(uint64_t k) {
  uint32_t b = (uint32_t)(k >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}
DEVI int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

// Top-k of one row of E logits by one wavefront, then the gate weights.
// Lane l holds the keys of experts l, l+64, ...; each round takes the
// wavefront maximum and the owning lane clears that key.  Lane r (< k) keeps
// rank r.  Gate weights: m = logit of rank 0, e_r = exp64(l_r - m), S = sum of
// e_r in rank order, w_r = fp32(e_r / S).  NPER >= ceil(E / 64).
template <int NPER, typename RowT>
DEVI void topk_wave(RowT row, int E, int k, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? sel_key(row(e), e) : 0ull;
  }
  float my_v = 0.f;
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    int e = key_index(best);
    if (best == 0ull || e < 0 || e >= E) e = 0;  // only with non-finite logits (out of contract)
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == r) {
      my_v = key_value(best);
      my_e = e;
    }
  }
  const double m = (double)__shfl(my_v, 0, 64);
  double ev = 0.0;
  if (lane < k) ev = moe_exp64((double)my_v - m);
  double S = 0.0;
  for (int r = 0; r < k; ++r) S += __shfl(ev, r, 64);  // rank order, same in every lane
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = (float)(ev / S);
  }
}

template <typename RowT>
DEVI void topk_wave_any(RowT row, int E, int k, int32_t* idx_out, float* w_out) {
  if (E <= 512) topk_wave<8>(row, E, k, idx_out, w_out);
  else if (E <= 1024) topk_wave<16>(row, E, k, idx_out, w_out);
  else if (E <= 2048) topk_wave<32>(row, E, k, idx_out, w_out);
  else topk_wave<64>(row, E, k, idx_out, w_out);
}

struct PtrRow {
  const float* p;
  DEVI float operator()(int e) const { return p[e]; }
};

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave_any(PtrRow{logits + (size_t)t * E}, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

// Sum 64 per-lane values across the wavefront so that lane l ends up with
// the total of value index l ("reduce-scatter"): at the step of distance h,
// a lane keeps the half of its values selected by its lane bit h and adds the
// partner's copy of that half.
DEVI float reduce_scatter64(float (&v)[64], int lane) {
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const bool up = (lane & h) != 0;
#pragma unroll
    for (int j = 0; j < h; ++j) {
      const float lo = v[j], hi = v[j + h];
      const float send = up ? lo : hi;
      const float keep = up ? hi : lo;
      v[j] = keep + __shfl_xor(send, h, 64);
    }
  }
  return v[0];
}

// ---------------------------------------------------------------------------
// Route: workgroup (column slice cs of 256 inputs, row slice rs of 64
// experts).  Sums the input splits for its columns, writes partial logits of
// its 64 experts over those columns; the rs == 0 workgroups also write the
// partial sums of squares, the summed input (if asked) and the fp16 hi/lo
// MFMA A-fragments of the 8 blocks of the slice:
//   lane L = m + 16q of block b holds row m (m < 8: token m, hi part; m >= 8:
//   token m-8, lo part) at inputs 8q..8q+7; xsum[b][m] = -code_off * sum.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ float ys[MOE_MAX_TOK_DECODE][MOE_ROUTE_COLS];
  const int cs = blockIdx.x, rs = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = a.T, d = a.d, E = a.E;
  const int c0 = cs * MOE_ROUTE_COLS;

  // router rows of this wave: issue the weight loads first (HBM latency)
  float4_t W4[16];
  const int e_base = rs * MOE_ROUTE_ROWS + wv * 16;
  if (a.do_logits) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = e_base + i;
      W4[i] = (e < E) ? __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(a.Wr + (size_t)e * d + c0) + lane)
                      : float4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  // summed input slice into LDS (splits added in order; all loads issued first)
  for (int i = tid; i < T * 64; i += 256) {
    const int t = i >> 6, c4 = i & 63;
    const float* src = a.in + (size_t)t * d + c0 + 4 * c4;
    float4_t v[MOE_MAX_IN_SPLITS];
#pragma unroll
    for (int s = 0; s < MOE_MAX_IN_SPLITS; ++s)
      v[s] = *reinterpret_cast<const float4_t*>(src + (size_t)(s < a.S_in ? s : 0) * a.in_stride);
    float4_t acc = v[0];
#pragma unroll
    for (int s = 1; s < MOE_MAX_IN_SPLITS; ++s)
      if (s < a.S_in) acc += v[s];
    *reinterpret_cast<float4_t*>(&ys[t][4 * c4]) = acc;
    if (rs == 0 && a.y_out) *reinterpret_cast<float4_t*>(a.y_out + (size_t)t * d + c0 + 4 * c4) = acc;
  }
  __syncthreads();

  if (rs == 0) {
    for (int t = wv; t < T; t += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&ys[t][4 * lane]);
      const float ss = wave_sum(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
      if (lane == 0) a.ss_part[cs * T + t] = ss;
    }
    const int m = lane & 15, q = lane >> 4, tok = m & 7, lo = m >> 3;
    for (int bl = wv; bl < MOE_ROUTE_COLS / 32; bl += 4) {
      const int b = cs * (MOE_ROUTE_COLS / 32) + bl;
      half8_t h;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float v = (tok < T) ? ys[tok][32 * bl + 8 * q + c] : 0.f;
        const _Float16 hi = (_Float16)v;
        const _Float16 out = lo ? (_Float16)(v - (float)hi) : hi;
        h[c] = out;
        s += (float)out;
      }
      *reinterpret_cast<half8_t*>(a.xfrag + ((size_t)b * 64 + lane) * 8) = h;
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (q == 0) a.xsum[b * 16 + m] = -(float)a.code_off * s;
    }
  }

  if (!a.do_logits) return;
  float4 y4[MOE_MAX_TOK_DECODE];
#pragma unroll
  for (int t = 0; t < MOE_MAX_TOK_DECODE; ++t)
    y4[t] = (t < T) ? *reinterpret_cast<const float4*>(&ys[t][4 * lane]) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float v[64];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float4_t w = W4[half * 8 + i];
        v[i * 8 + t] = w.x * y4[t].x + w.y * y4[t].y + w.z * y4[t].z + w.w * y4[t].w;
      }
    const float s = reduce_scatter64(v, lane);
    const int e = e_base + half * 8 + (lane >> 3), t = lane & 7;
    if (e < E && t < T) a.lp[((size_t)cs * T + t) * E + e] = s;
  }
}

// ---------------------------------------------------------------------------
// Select: one workgroup per token.  Sums the token's partial logits in
// column-slice order (every load issued before the first add), applies 1/rms
// and the bias, and wavefront 0 selects the top-k and the gate weights.  With
// forced routing it only copies the given row.  The slot list is built by
// the expert kernels themselves.
// ---------------------------------------------------------------------------
template <int MAXCS>
DEVI void sum_partials(const SelectArgs& a, int t, float den, float* row) {
  const int tid = threadIdx.x, T = a.T, E = a.E, n_cs = a.n_cs;
  for (int e0 = 0; e0 < E; e0 += 512) {
    float tmp[2][MAXCS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = min(e0 + tid + 256 * j, E - 1);
#pragma unroll
      for (int c = 0; c < MAXCS; ++c) tmp[j][c] = a.lp[((size_t)min(c, n_cs - 1) * T + t) * E + e];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + tid + 256 * j;
      float acc = tmp[j][0];
#pragma unroll
      for (int c = 1; c < MAXCS; ++c)
        if (c < n_cs) acc += tmp[j][c];
      if (e < E) {
        const float l = (a.norm ? acc / den : acc) + a.br[e];
        row[e] = l;
        a.logits[(size_t)t * E + e] = l;
        if (a.out_logits) a.out_logits[(size_t)t * E + e] = l;
      }
    }
  }
}

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  extern __shared__ float row[];  // [E]
  __shared__ float den_s;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = a.T, k = a.k;
  if (wv == 0) {
    float v = (a.norm && lane < a.n_cs) ? a.ss_part[lane * T + t] : 0.f;
    v = wave_sum(v);
    if (lane == 0) {
      const float r = a.norm ? sqrtf(v / (float)a.d + a.eps) : 1.0f;
      den_s = r;
      a.rnorm[t] = r;
    }
  }
  if (a.fidx) {
    if (tid < k) {
      const int32_t e = a.fidx[t * k + tid];
      const float w = a.fw[t * k + tid];
      a.idx[t * k + tid] = e;
      a.w[t * k + tid] = w;
      if (a.out_idx) a.out_idx[t * k + tid] = e;
      if (a.out_w) a.out_w[t * k + tid] = w;
    }
    return;
  }
  __syncthreads();
  const float den = den_s;
  if (a.n_cs <= 16) sum_partials<16>(a, t, den, row);
  else sum_partials<32>(a, t, den, row);
  __syncthreads();
  if (wv == 0) {
    topk_wave_any(PtrRow{row}, a.E, k, a.idx + t * k, a.w + t * k);
    if (lane < k) {
      if (a.out_idx) a.out_idx[t * k + lane] = a.idx[t * k + lane];
      if (a.out_w) a.out_w[t * k + lane] = a.w[t * k + lane];
    }
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int S, int64_t stride, int n4,
                                                      float* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4_t v[MOE_MAX_IN_SPLITS];
#pragma unroll
  for (int s = 0; s < MOE_MAX_IN_SPLITS; ++s)
    v[s] = *reinterpret_cast<const float4_t*>(part + (size_t)(s < S ? s : 0) * stride + 4 * (size_t)i);
  float4_t acc = v[0];
#pragma unroll
  for (int s = 1; s < MOE_MAX_IN_SPLITS; ++s)
    if (s < S) acc += v[s];
  reinterpret_cast<float4_t*>(y)[i] = acc;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int d, float eps,
                                                      float* __restrict__ y) {
  __shared__ float part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)t * d;
  float ss = 0.f;
  for (int j = tid * 4; j < d; j += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + j);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float dn = sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
  for (int j = tid * 4; j < d; j += 1024) {
    float4 v = *reinterpret_cast<const float4*>(xr + j);
    v.x /= dn; v.y /= dn; v.z /= dn; v.w /= dn;
    *reinterpret_cast<float4*>(y + (size_t)t * d + j) = v;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const dim3 grid(a.d / MOE_ROUTE_COLS, a.do_logits ? (a.E + MOE_ROUTE_ROWS - 1) / MOE_ROUTE_ROWS : 1);
  hipLaunchKernelGGL(route_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const size_t lds = sizeof(float) * (size_t)a.E;
  hipLaunchKernelGGL(select_kernel, dim3(a.T), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part, int S, int64_t stride, int T, int d, float* y, hipStream_t s) {
  const int n4 = T * d / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((n4 + 255) / 256), dim3(256), 0, s, part, S, stride, n4, y);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int T, int d, float eps, float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, s, x, d, eps, y);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t moe_route_kernels_init() { return hipSuccess; }
