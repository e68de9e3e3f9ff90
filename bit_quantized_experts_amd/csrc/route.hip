// route.hip -- router GEMV, top-k selection with gate weights, the expert
// slot list for the decode kernels, RMSNorm between stacked layers.
//
// The router keeps about ten of 512 small experts per token [cnyes profile of
// Strata, section "Strata 到底是什麼？"]; it stays resident next to the
// shared expert [same page, section "三層記憶體", part 1].
#include "kern_common.h"
#include "moe_launch.h"

namespace {

// (v, e) ranks before (bv, be): larger logit, or equal logit and lower index.
DEVI bool ranks_before(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }

// Top-k of one row of E logits by one wavefront, then the gate weights.
// Selection is done k times; round r takes the best item that ranks strictly
// after the item taken in round r-1 (order: logit descending, index
// ascending), so no "taken" marks are needed.  The row is read through `row`
// (global or LDS).  Lane r (< k) ends up owning rank r.
// Gate weights: m = logit of rank 0, e_r = exp64(l_r - m), S = sum of e_r in
// rank order (one lane, sequentially), w_r = fp32(e_r / S).
template <typename RowT>
DEVI void topk_wave(RowT row, int E, int k, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  float pv = __builtin_inff();
  int pe = -1;
  float my_v = 0.f;
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
    for (int e = lane; e < E; e += 64) {
      const float v = row(e);
      const bool elig = (v < pv) || (v == pv && e > pe);
      if (elig && ranks_before(v, e, bv, be)) { bv = v; be = e; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ranks_before(ov, oe, bv, be)) { bv = ov; be = oe; }
    }
    if (be < 0 || be >= E) be = 0;  // only with non-finite logits (out of contract): stay in range
    if (lane == r) { my_v = bv; my_e = be; }
    pv = bv;
    pe = be;
  }
  const double m = (double)__shfl(my_v, 0, 64);
  double ev = 0.0;
  if (lane < k) ev = moe_exp64((double)my_v - m);
  double S = 0.0;
  for (int r = 0; r < k; ++r) S += __shfl(ev, r, 64);  // same order in every lane
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = (float)(ev / S);
  }
}

struct GlobalRow {
  const float* p;
  DEVI float operator()(int e) const { return p[e]; }
};
struct LdsRow {
  const float* p;
  DEVI float operator()(int e) const { return p[e]; }
};

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave(GlobalRow{logits + (size_t)t * E}, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------------------
// Decode route kernel (T <= 8).  Every workgroup: (optionally) RMSNorm the
// input rows into LDS, compute the logits of its slice of experts, and write
// its share of the fp16 hi/lo MFMA fragments of x.  The last workgroup to
// finish (device-scope counter) selects the top-k per token and builds the
// slot list: distinct routed experts in ascending id order, then the shared
// expert, with per-token gate weights per slot (0 = token not routed there).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_decode_kernel(RouteArgs a) {
  extern __shared__ float lds[];  // [max(T*d, T*E, ...)] floats
  __shared__ float den[MOE_MAX_TOK_DECODE];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = a.T, d = a.d, E = a.E;

  // 1. normalisation factors (each workgroup computes them for itself)
  if (a.norm) {
    for (int t = wv; t < T; t += 4) {
      float ss = 0.f;
      for (int j = lane * 4; j < d; j += 256) {
        const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)t * d + j);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = wave_sum(ss);
      if (lane == 0) den[t] = sqrtf(ss / (float)d + a.eps);
    }
  }
  __syncthreads();
  // 2. input rows into LDS
  for (int i = tid * 4; i < T * d; i += 1024) {
    float4 v = *reinterpret_cast<const float4*>(a.x + i);
    if (a.norm) {
      const float dn = den[i / d];
      v.x /= dn; v.y /= dn; v.z /= dn; v.w /= dn;
    }
    *reinterpret_cast<float4*>(lds + i) = v;
  }
  __syncthreads();

  // 3. logits of this workgroup's experts, one wavefront per expert row
  if (!a.fidx) {
    const int e0 = blockIdx.x * a.rows_per_wg;
    const int e1 = min(E, e0 + a.rows_per_wg);
    for (int e = e0 + wv; e < e1; e += 4) {
      float acc[MOE_MAX_TOK_DECODE];
#pragma unroll
      for (int t = 0; t < MOE_MAX_TOK_DECODE; ++t) acc[t] = 0.f;
      const float* wr = a.Wr + (size_t)e * d;
      for (int j = lane * 4; j < d; j += 256) {
        const float4 w4 = *reinterpret_cast<const float4*>(wr + j);
#pragma unroll
        for (int t = 0; t < MOE_MAX_TOK_DECODE; ++t) {
          if (t < T) {
            const float4 x4 = *reinterpret_cast<const float4*>(lds + t * d + j);
            acc[t] += w4.x * x4.x + w4.y * x4.y + w4.z * x4.z + w4.w * x4.w;
          }
        }
      }
      const float b = a.br[e];
#pragma unroll
      for (int t = 0; t < MOE_MAX_TOK_DECODE; ++t) {
        if (t < T) {
          const float s = wave_sum(acc[t]) + b;
          if (lane == 0) {
            a.logits[(size_t)t * E + e] = s;
            if (a.out_logits) a.out_logits[(size_t)t * E + e] = s;
          }
        }
      }
    }
  }

  // 4. x as fp16 hi/lo MFMA A-fragments: lane l = m + 16q holds row m (token m
  //    for m < 8 as the hi part, token m-8 as the lo part) at inputs 8q..8q+7
  //    of the block; xsum[b][m] = -code_off * (sum of those 32 fp16 values).
  {
    const int nb = d / 32;
    const int gw = blockIdx.x * 4 + wv, nwt = gridDim.x * 4;
    const int m = lane & 15, q = lane >> 4, tok = m & 7, lo = m >> 3;
    for (int b = gw; b < nb; b += nwt) {
      half8_t h;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float v = (tok < T) ? lds[tok * d + 32 * b + 8 * q + c] : 0.f;
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

  // 5. last workgroup: top-k and slot list
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const uint32_t old = atomicAdd(a.counter, 1u);
    is_last = (old == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  const int k = a.k;
  if (a.fidx) {
    for (int i = tid; i < T * k; i += 256) {
      a.idx[i] = a.fidx[i];
      a.w[i] = a.fw[i];
    }
  } else {
    // logits of all experts into LDS (x is no longer needed)
    __syncthreads();
    for (int i = tid; i < T * E; i += 256) lds[i] = __builtin_nontemporal_load(a.logits + i);
    __syncthreads();
    for (int t = wv; t < T; t += 4) topk_wave(LdsRow{lds + t * E}, E, k, a.idx + t * k, a.w + t * k);
  }
  __syncthreads();
  __threadfence_block();

  // slot list: mark routed experts, compact in ascending id order
  int* mark = reinterpret_cast<int*>(lds);  // [E]
  __shared__ int wave_tot[4];
  __shared__ int n_routed;
  __syncthreads();
  for (int e = tid; e < E; e += 256) mark[e] = 0;
  __syncthreads();
  for (int i = tid; i < T * k; i += 256) {
    const int e = a.idx[i];
    if (e >= 0 && e < E) mark[e] = 1;
  }
  __syncthreads();
  const int per = (E + 255) / 256;
  const int e_beg = min(E, tid * per), e_end = min(E, e_beg + per);
  int cnt = 0;
  for (int e = e_beg; e < e_end; ++e) cnt += mark[e];
  int incl = cnt;  // inclusive scan within the wavefront
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wv; ++i) base += wave_tot[i];
  int pos = base + incl - cnt;
  for (int e = e_beg; e < e_end; ++e) {
    if (mark[e]) {
      a.slot_expert[pos] = e;
      mark[e] = pos + 1;
      ++pos;
    }
  }
  if (tid == 255) n_routed = base + incl;
  __syncthreads();
  const int nr = n_routed;
  const int ns = nr + (a.has_shared ? 1 : 0);
  for (int i = tid; i < ns * 8; i += 256) a.slot_w[i] = 0.f;
  __syncthreads();
  for (int i = tid; i < T * k; i += 256) {
    const int e = a.idx[i];
    if (e >= 0 && e < E) a.slot_w[(mark[e] - 1) * 8 + i / k] = a.w[i];
  }
  if (a.has_shared && tid < T) a.slot_w[nr * 8 + tid] = 1.0f;
  if (tid == 0) {
    if (a.has_shared) a.slot_expert[nr] = E;
    *a.n_slots = ns;
    *a.counter = 0u;
  }
  for (int i = tid; i < T * k; i += 256) {
    if (a.out_idx) a.out_idx[i] = a.idx[i];
    if (a.out_w) a.out_w[i] = a.w[i];
  }
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

hipError_t launch_route_decode(const RouteArgs& a, int n_wg, hipStream_t s) {
  size_t lds = sizeof(float) * (size_t)a.T * (size_t)(a.d > a.E ? a.d : a.E);
  if (lds < sizeof(int) * (size_t)a.E) lds = sizeof(int) * (size_t)a.E;
  hipLaunchKernelGGL(route_decode_kernel, dim3(n_wg), dim3(256), lds, s, a);
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

hipError_t moe_route_kernels_init() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&route_decode_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
}
