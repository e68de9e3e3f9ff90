// route.hip -- router GEMV, top-k selection with gate weights, the expert
// slot list for the decode kernels, RMSNorm between stacked layers.
//
// The router keeps about ten of 512 small experts per token [cnyes profile of
// Strata, section "Strata 到底是什麼？"]; it stays resident next to the
// shared expert [same page, section "三層記憶體", part 1].
//
// Decode (T <= 8) splits the router GEMV over column slices of the input so
// that no workgroup needs the whole input row: the previous layer's output
// arrives as split partial sums, and each workgroup adds only the 128 columns
// it multiplies.  RMSNorm is a per-token scale, so it is applied after the
// dot products (logit = (y . w) / rms(y) + bias) and, in the expert kernels,
// to the accumulators before the SwiGLU nonlinearity.
#include "kern_common.h"
#include "moe_launch.h"
#include "topk.h"

namespace {

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
// Logits, finished inside the route kernel by the workgroup of each row slice
// that completes last (no workgroup waits for another): every workgroup,
// once its partial logits and its sums of squares are stored, counts itself
// on the counter of its row slice rs; the one that completes the count (the
// last of the n_cs column slices) forms, for the slice's 64 experts and
// every token, the sum of the partial logits in column-slice order times the
// router row factor 2^ew (exact), the token's divisor r = sqrt(sum of
// squares / d + eps) (1 without the norm; the slice's own copies of the sums
// of squares, added in column-slice order, so every slice gets the same r),
// and the logit (sum / r) + bias.  It puts the counter back to zero for the
// next call.  The top-k selection is left to the gate/up kernel.
//
// The values handed between workgroups (partial logits, sums of squares)
// are stored and loaded device-coherently (agent-scope relaxed atomics: sc1
// accesses that no workgroup's L2 keeps stale), so the count needs no cache
// write-back or invalidation, only the wait for the stores.
// ---------------------------------------------------------------------------
DEVI void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEVI float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts the calling workgroup on *ctr once all its device-coherent stores
// have completed; true in every thread of the workgroup that completes
// `total`, which then sees every counted workgroup's stores.
DEVI bool count_done(uint32_t* ctr, uint32_t total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1u;
  __syncthreads();
  return *flag != 0;
}

// Wavefront wv finishes tokens wv + 4j (below T), two at a time (pairs p =
// tid and tid + 256 of a pass: token 8h + p / 64, expert rs * 64 + p % 64);
// every load of a pass is issued before its first add, at clamped
// addresses.
template <int MAXCS>
DEVI void finish_slice(const RouteArgs& a, int rs) {
  const SelectArgs& c = a.sel;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = a.T, E = a.E, n_cs = c.n_cs;
  static_assert(MOE_MAX_TOK_F16ACT <= 16, "two passes of 8 tokens");
  const int er = rs * MOE_ROUTE_ROWS + lane, e = min(er, E - 1);
  const bool e_ok = er < E;
  const int ew = a.do_logits ? c.ew[e] : 0;
  const float bias = a.do_logits ? c.br[e] : 0.f;
  const float* ssr = c.ss_part + (size_t)rs * n_cs * T;
  for (int h = 0; 8 * h < T; ++h) {
    int t[2];
    float ss[2], tmp[2][MAXCS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      t[j] = min(8 * h + wv + 4 * j, T - 1);
      ss[j] = ld_dev(ssr + min(lane, n_cs - 1) * T + t[j]);
      if (a.do_logits) {
#pragma unroll
        for (int q = 0; q < MAXCS; ++q) tmp[j][q] = ld_dev(a.lp + ((size_t)min(q, n_cs - 1) * T + t[j]) * E + e);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tok = 8 * h + wv + 4 * j;
      const float r = c.norm ? sqrtf(wave_sum((lane < n_cs) ? ss[j] : 0.f) / (float)c.d + c.eps) : 1.0f;
      if (tok >= T) continue;
      if (rs == 0 && lane == 0) c.rnorm[tok] = r;
      if (!a.do_logits) continue;
      float acc = tmp[j][0];
#pragma unroll
      for (int q = 1; q < MAXCS; ++q)
        if (q < n_cs) acc += tmp[j][q];
      const float x = ldexpf(acc, ew);  // router row factor, exact
      const float l = (c.norm ? x / r : x) + bias;
      if (e_ok) {
        c.logits[(size_t)tok * E + er] = l;
        if (c.out_logits) c.out_logits[(size_t)tok * E + er] = l;
      }
    }
  }
}

DEVI void route_finish(const RouteArgs& a, int rs) {
  __shared__ int flag;
  if (!count_done(a.sel.ctrl + rs, (uint32_t)a.sel.n_cs, &flag)) return;
  if (threadIdx.x == 0) a.sel.ctrl[rs] = 0u;
  if (a.sel.n_cs <= 16) finish_slice<16>(a, rs);
  else if (a.sel.n_cs <= 20) finish_slice<20>(a, rs);  // d = 2560
  else if (a.sel.n_cs <= 32) finish_slice<32>(a, rs);
  else finish_slice<64>(a, rs);
}

// ---------------------------------------------------------------------------
// Route: workgroup (column slice cs of 128 inputs, row slice rs of 64
// experts).  Sums the input splits for its columns, writes partial logits of
// its 64 experts over those columns and the slice's sums of squares (every
// row slice its own copy); the rs == 0 workgroups also write the summed input
// (if asked) and the fp16 hi/lo MFMA A-fragments of the 4 blocks of the
// slice:
//   lane L = m + 16q of block b holds row m (m < 8: token m, hi part; m >= 8:
//   token m-8, lo part) at inputs 8q..8q+7; xsum[b][m] = -code_off * sum;
//   with fp16 activations (act16) row m is token m rounded to fp16.
// The partial logits run on the matrix cores: hi/lo A-fragments of 8 tokens
// (built in registers by every workgroup; a second row tile for tokens 8..15)
// times the router rows prepared at pack time
// as 2^ew (wh + wl), fp16 hi and lo B-fragments, so one wavefront's 16
// experts over the 4 blocks take 8 v_mfma_f32_16x16x32_f16 and the hi and lo
// rows of a token are added once at the end.  All four products of the
// ~22-bit operands are formed exactly; the rounding is fp32 accumulation.
// The power of two 2^ew of each router row is applied to the summed
// partials (exact) by the workgroup that finishes the row slice (above).
// ---------------------------------------------------------------------------
DEVI half8_t x_fragment(const float (*ys)[MOE_ROUTE_COLS], int bl, int lane, int T, float* sum) {
  const int m = lane & 15, q = lane >> 4, tok = m & 7, lo = m >> 3;  // (ys, T: from the tile's first token)
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

// The same block with one fp16 row per token (16 tokens).
DEVI half8_t x_fragment16(const float (*ys)[MOE_ROUTE_COLS], int bl, int lane, int T, float* sum) {
  const int m = lane & 15, q = lane >> 4;
  float4_t v0 = float4_t{0.f, 0.f, 0.f, 0.f}, v1 = v0;
  if (m < T) {
    v0 = *reinterpret_cast<const float4_t*>(&ys[m][32 * bl + 8 * q]);
    v1 = *reinterpret_cast<const float4_t*>(&ys[m][32 * bl + 8 * q + 4]);
  }
  half8_t h;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    h[c] = (_Float16)(c < 4 ? v0[c] : v1[c - 4]);
    s += (float)h[c];
  }
  *sum = s;
  return h;
}

__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ float ys[MOE_MAX_TOK_F16ACT][MOE_ROUTE_COLS];
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
  constexpr int RQ = MOE_ROUTE_COLS / 4;                   // float4 per token row of the slice
  constexpr int PER = (MOE_MAX_TOK_F16ACT * RQ + 255) / 256;  // float4 per thread
  float4_t v[PER][MOE_MAX_IN_SPLITS];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + 256 * j, t = min(i / RQ, T - 1), c4 = i % RQ;  // (rows past T re-read row T - 1)
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
    const int i = tid + 256 * j, t = i / RQ, c4 = i % RQ;
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

  // sums of squares of the slice (each row slice keeps its own copy)
  for (int t = wv; t < T; t += 4) {
    const float4 v = lane < RQ ? *reinterpret_cast<const float4*>(&ys[t][4 * lane]) : float4{0.f, 0.f, 0.f, 0.f};
    const float ss = wave_sum(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
    if (lane == 0) st_dev(a.sel.ss_part + ((size_t)rs * gridDim.x + cs) * T + t, ss);
  }
  if (rs == 0) {
    const int m = lane & 15, q = lane >> 4;
    for (int bl = wv; bl < NBL; bl += 4) {
      const int b = cs * NBL + bl;
      float s;
      const half8_t h = a.act16 ? x_fragment16(ys, bl, lane, T, &s) : x_fragment(ys, bl, lane, T, &s);
      *reinterpret_cast<half8_t*>(a.xfrag + ((size_t)b * 64 + lane) * 8) = h;
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (q == 0) a.xsum[b * 16 + m] = -(float)a.code_off * s;
    }
  }

  if (tile_ok) {
    // row tiles of 8 tokens: tokens 8 tb .. 8 tb + 7
    for (int tb = 0; 8 * tb < T; ++tb) {
      half8_t A[NBL];
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        float s;
        A[j] = x_fragment(ys + 8 * tb, j, lane, T - 8 * tb, &s);
      }
      float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        acc = mfma16x16x32(A[j], BH[j], acc);
        acc = mfma16x16x32(A[j], BL[j], acc);
      }
      // lane l: expert et*16 + (l & 15), C rows 4(l>>4)+i: token 8 tb +
      // 4((l>>4)&1)+i, hi part in lanes < 32, lo part in lanes >= 32.  The
      // partial logits are left without the row factor 2^ew; it is applied
      // to their sum.
      const int e = et * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = add_partner32(acc[i]);
        const int t = 8 * tb + 4 * ((lane >> 4) & 1) + i;
        if (lane < 32 && e < E && t < T) st_dev(a.lp + ((size_t)cs * T + t) * E + e, v);
      }
    }
  }
  route_finish(a, rs);
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
  // the completion counts must match the grid, or no workgroup selects
  if ((int)grid.x != a.sel.n_cs || (int)grid.y != a.sel.n_rs || a.sel.n_rs > MOE_CTRL_WORDS ||
      a.sel.n_cs > MOE_MAX_CS || a.T < 1 || a.T > (a.act16 ? MOE_MAX_TOK_F16ACT : MOE_MAX_TOK_DECODE))
    return hipErrorInvalidValue;
  MOE_LAUNCH(route_kernel, grid, dim3(256), 0, s, a);
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
