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
// Lane l holds the keys of experts l, l+64, ...; keys are unique.
//   1. Candidates: theta = the k-th largest of the 64 lane maxima (ranked by
//      counting larger maxima through LDS).  At least k keys are >= theta
//      (those k maxima), and every key of the top k is >= theta.
//   2. If at most 64 keys are >= theta they are compacted to LDS, each is
//      ranked by counting the larger candidates, and the first k ranks are
//      the answer.  Otherwise (many equal logits) a radix search on the value
//      keys finds the k-th largest value (a trial threshold is kept while at
//      least k values reach it, stopping once exactly k do); the values above
//      it and the tied ones in ascending expert index are taken, compacted
//      and ranked the same way.
// Lane r ends up with rank r (value descending, then index ascending).  Gate
// weights: m = logit of rank 0, e_r = exp64(l_r - m), S = sum of e_r in rank
// order, w_r = fp32(e_r / S).  `buf`: this wave's 96 LDS entries.  NPER >=
// ceil(E / 64).
DEVI int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

DEVI double readlane_f64(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

DEVI uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int TOPK_BUF = 96;  // LDS entries per wave: 64 candidates + 32

template <int NPER, typename RowT>
DEVI void topk_wave(RowT row, int E, int k, int32_t* idx_out, float* w_out, uint64_t* buf) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NPER];
  uint64_t lmax = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? sel_key(row(e), e) : 0ull;  // 0: no expert
    lmax = key[i] > lmax ? key[i] : lmax;
  }
  // 1. theta = k-th largest lane maximum
  buf[lane] = lmax;
  int rk = 0;
  for (int j = 0; j < 64; ++j) rk += (buf[j] > lmax) ? 1 : 0;
  const uint64_t at = __ballot(rk == k - 1 && lmax != 0ull);
  const uint64_t theta = readlane_u64(lmax, at ? (int)__builtin_ctzll(at) : 0);
  int c = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) c += (int)__builtin_popcountll(__ballot(key[i] >= theta));

  // 2. choose the candidate set: keys >= theta, or the exact top k
  bool exact = true;
  uint32_t tau = 0;
  int need = 0;
  if (c > 64) {
    uint32_t hv[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) hv[i] = (uint32_t)(key[i] >> 32);
    exact = false;
    for (int b = 31; b >= 0; --b) {
      const uint32_t t = tau | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) cnt += (int)__builtin_popcountll(__ballot(hv[i] >= t));
      if (cnt >= k) {
        tau = t;
        if (cnt == k) {
          exact = true;
          break;
        }
      }
    }
    if (!exact) {
      int c_gt = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) c_gt += (int)__builtin_popcountll(__ballot(hv[i] > tau));
      need = k - c_gt;
    }
  }
  const bool radix = c > 64;
  // compact the candidates to buf[0..n) in (slot, lane) order
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const uint32_t hv = (uint32_t)(key[i] >> 32);
    bool take;
    if (!radix) {
      take = key[i] >= theta;
    } else {
      const bool tie = !exact && hv == tau;
      const uint64_t tm = __ballot(tie);
      take = exact ? (hv >= tau) : (hv > tau || (tie && lanes_below(tm) < need));
      need -= min(need, (int)__builtin_popcountll(tm));
    }
    const uint64_t sm = __ballot(take);
    const int pos = n + lanes_below(sm);
    if (take && pos < 64) buf[pos] = key[i];
    n += (int)__builtin_popcountll(sm);
  }
  n = min(n, 64);
  // rank the candidates; the first k ranks are the result
  const uint64_t mine = (lane < n) ? buf[lane] : 0ull;
  int rank = 0;
  for (int j = 0; j < n; ++j) rank += (buf[j] > mine) ? 1 : 0;
  if (lane < n && rank < k) buf[64 + rank] = mine;
  const uint64_t kr = (lane < k) ? buf[64 + lane] : 0ull;
  const float my_v = key_value(kr);
  const int my_e = key_index(kr);
  const double m = (double)__builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, my_v)));
  double ev = 0.0;
  if (lane < k) ev = moe_exp64((double)my_v - m);
  double S = 0.0;
  for (int r = 0; r < k; ++r) S += readlane_f64(ev, r);  // rank order, same in every lane
  if (lane < k) {
    idx_out[lane] = (my_e >= 0 && my_e < E) ? my_e : 0;  // (other only with non-finite logits, out of contract)
    w_out[lane] = (float)(ev / S);
  }
}

template <typename RowT>
DEVI void topk_wave_any(RowT row, int E, int k, int32_t* idx_out, float* w_out, uint64_t* buf) {
  if (E <= 512) topk_wave<8>(row, E, k, idx_out, w_out, buf);
  else if (E <= 1024) topk_wave<16>(row, E, k, idx_out, w_out, buf);
  else if (E <= 2048) topk_wave<32>(row, E, k, idx_out, w_out, buf);
  else topk_wave<64>(row, E, k, idx_out, w_out, buf);
}

struct PtrRow {
  const float* p;
  DEVI float operator()(int e) const { return p[e]; }
};

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ uint64_t buf[4][TOPK_BUF];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave_any(PtrRow{logits + (size_t)t * E}, E, k, idx + (size_t)t * k, w + (size_t)t * k, buf[threadIdx.x >> 6]);
}

// ---------------------------------------------------------------------------
// Route: workgroup (column slice cs of 256 inputs, row slice rs of 64
// experts).  Sums the input splits for its columns, writes partial logits of
// its 64 experts over those columns; the rs == 0 workgroups also write the
// partial sums of squares, the summed input (if asked) and the fp16 hi/lo
// MFMA A-fragments of the 8 blocks of the slice:
//   lane L = m + 16q of block b holds row m (m < 8: token m, hi part; m >= 8:
//   token m-8, lo part) at inputs 8q..8q+7; xsum[b][m] = -code_off * sum.
// The partial logits run on the matrix cores: the same A-fragments (built in
// registers by every workgroup) times the router rows prepared at pack time
// as 2^ew (wh + wl), fp16 hi and lo B-fragments, so one wavefront's 16
// experts over the 8 blocks take 16 v_mfma_f32_16x16x32_f16 and the hi and lo
// rows of a token are added once at the end.  All four products of the
// ~22-bit operands are formed exactly; the rounding is fp32 accumulation.
// The power of two 2^ew of each router row is applied by the select kernel
// to the summed partials (exact).
// ---------------------------------------------------------------------------
DEVI half8_t x_fragment(const float (*ys)[MOE_ROUTE_COLS], int bl, int lane, int T, float* sum) {
  const int m = lane & 15, q = lane >> 4, tok = m & 7, lo = m >> 3;
  float4_t v0 = float4_t{0.f, 0.f, 0.f, 0.f}, v1 = v0;
  if (tok < T) {
    v0 = *reinterpret_cast<const float4_t*>(&ys[tok][32 * bl + 8 * q]);
    v1 = *reinterpret_cast<const float4_t*>(&ys[tok][32 * bl + 8 * q + 4]);
  }
  half8_t h;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float v = c < 4 ? v0[c] : v1[c - 4];
    const _Float16 hi = (_Float16)v;
    const _Float16 out = lo ? (_Float16)(v - (float)hi) : hi;
    h[c] = out;
    s += (float)out;
  }
  *sum = s;
  return h;
}

__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ float ys[MOE_MAX_TOK_DECODE][MOE_ROUTE_COLS];
  const int cs = blockIdx.x, rs = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, d = a.d, E = a.E;
  const int c0 = cs * MOE_ROUTE_COLS;
  constexpr int NBL = MOE_ROUTE_COLS / 32;  // blocks per column slice

  // the input splits of this slice first (the previous kernel's output), then
  // the router fragments of this wave's 16 experts and their row exponents:
  // the wait for the inputs leaves the router loads in flight
  // (every load is issued, rows past T and splits past S_in re-read a valid
  // address, so the wait counts before the first add are exact)
  const int et = rs * (MOE_ROUTE_ROWS / 16) + wv;  // 16-expert tile
  const bool tile_ok = a.do_logits && et * 16 < E;
  constexpr int PER = MOE_MAX_TOK_DECODE * 64 / 256;  // float4 per thread
  float4_t v[PER][MOE_MAX_IN_SPLITS];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + 256 * j, t = min(i >> 6, T - 1), c4 = i & 63;
    const float* src = a.in + (size_t)t * d + c0 + 4 * c4;
#pragma unroll
    for (int s = 0; s < MOE_MAX_IN_SPLITS; ++s)
      v[j][s] = *reinterpret_cast<const float4_t*>(src + (size_t)min(s, a.S_in - 1) * a.in_stride);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the input loads ahead of the router loads
  // (issued by every wave, tile 0 standing in for a wave without a tile, so
  // the wait counts stay exact)
  half8_t BH[NBL], BL[NBL];
  {
    const size_t base = ((size_t)(tile_ok ? et : 0) * (d / 32) + cs * NBL) * 64 * 8;
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      BH[j] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(a.wh + base + ((size_t)j * 64 + lane) * 8));
      BL[j] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(a.wl + base + ((size_t)j * 64 + lane) * 8));
    }
  }
  // summed input slice into LDS (splits added in order)
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + 256 * j, t = i >> 6, c4 = i & 63;
    if (t < T) {
      float4_t acc = v[j][0];
#pragma unroll
      for (int s = 1; s < MOE_MAX_IN_SPLITS; ++s)
        if (s < a.S_in) acc += v[j][s];
      *reinterpret_cast<float4_t*>(&ys[t][4 * c4]) = acc;
      if (rs == 0 && a.y_out) *reinterpret_cast<float4_t*>(a.y_out + (size_t)t * d + c0 + 4 * c4) = acc;
    }
  }
  __syncthreads();

  if (rs == 0) {
    for (int t = wv; t < T; t += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&ys[t][4 * lane]);
      const float ss = wave_sum(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
      if (lane == 0) a.ss_part[cs * T + t] = ss;
    }
    const int m = lane & 15, q = lane >> 4;
    for (int bl = wv; bl < NBL; bl += 4) {
      const int b = cs * NBL + bl;
      float s;
      const half8_t h = x_fragment(ys, bl, lane, T, &s);
      *reinterpret_cast<half8_t*>(a.xfrag + ((size_t)b * 64 + lane) * 8) = h;
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (q == 0) a.xsum[b * 16 + m] = -(float)a.code_off * s;
    }
  }

  if (!tile_ok) return;
  half8_t A[NBL];
#pragma unroll
  for (int j = 0; j < NBL; ++j) {
    float s;
    A[j] = x_fragment(ys, j, lane, T, &s);
  }
  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NBL; ++j) {
    acc = mfma16x16x32(A[j], BH[j], acc);
    acc = mfma16x16x32(A[j], BL[j], acc);
  }
  // lane l: expert et*16 + (l & 15), C rows 4(l>>4)+i: token 4((l>>4)&1)+i,
  // hi part in lanes < 32, lo part in lanes >= 32.  The partial logits are
  // left without the row factor 2^ew; the select kernel applies it to the sum.
  const int e = et * 16 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = add_partner32(acc[i]);
    const int t = 4 * ((lane >> 4) & 1) + i;
    if (lane < 32 && e < E && t < T) a.lp[((size_t)cs * T + t) * E + e] = v;
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
    float tmp[2][MAXCS], bias[2];
    int ew[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // bias and row exponent first: they wait for nothing
      const int e = min(e0 + tid + 256 * j, E - 1);
      bias[j] = a.br[e];
      ew[j] = a.ew[e];
    }
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
        const float x = ldexpf(acc, ew[j]);  // router row factor, exact
        const float l = (a.norm ? x / den : x) + bias[j];
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
  __shared__ uint64_t tk_buf[TOPK_BUF];
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
    topk_wave_any(PtrRow{row}, a.E, k, a.idx + t * k, a.w + t * k, tk_buf);
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
  MOE_LAUNCH(route_kernel, grid, dim3(256), 0, s, a);
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
