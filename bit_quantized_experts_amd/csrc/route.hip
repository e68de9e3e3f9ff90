// route.hip -- the decode router as its own kernel (route_dev.h), the
// standalone top-k selection, RMSNorm, the combine of split partial sums and
// a fill kernel.
#include "route_dev.h"
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

// Split prefill router (short chunks), E <= 512: a token's partial sums
// over the 256-column slices added in slice order from zero, scaled and
// biased (the steps of the separate reduce kernel), written out, and the
// token's top k taken from the wavefront's registers (as topk_kernel takes
// it from memory); one wavefront per token, every load in flight at once.
template <int MAXNS>
__global__ __launch_bounds__(256) void pf_router_topk_kernel(PfRouterArgs a, int k, int32_t* __restrict__ idx,
                                                             float* __restrict__ w) {
  constexpr int NPER = 8;
  __shared__ uint64_t buf[4][TOPK_BUF];
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6)), lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int E = a.E, ns = a.d / 256;
  float v[NPER][MAXNS];
  int ewv[NPER];
  float bv[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = min(lane + 64 * i, E - 1);
#pragma unroll
    for (int z = 0; z < MAXNS; ++z) v[i][z] = a.part[((size_t)min(z, ns - 1) * a.T + t) * E + e];
    ewv[i] = a.ew[e];
    bv[i] = a.bias[e];
  }
  const int ext = a.ex[t];
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    float tot = 0.f;
#pragma unroll
    for (int z = 0; z < MAXNS; ++z)
      if (z < ns) tot += v[i][z];
    const float l = ldexpf(tot, ext + ewv[i]) + bv[i];
    key[i] = 0ull;  // 0: no expert
    if (e < E) {
      a.logits[(size_t)t * E + e] = l;
      key[i] = sel_key(l, e);
    }
  }
  topk_keys<NPER>(key, E, k, idx + (size_t)t * k, w + (size_t)t * k, buf[threadIdx.x >> 6]);
}

__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ float ys[MOE_MAX_TOK_F16ACT][MOE_ROUTE_COLS];
  __shared__ int xe[MOE_MAX_TOK_F16ACT];  // slice exponent of each token
  __shared__ int flag;
  route_role<false>(a, blockIdx.x, blockIdx.y, ys, xe, &flag, nullptr, 0u, nullptr, nullptr);
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
      a.sel.n_cs > MOE_MAX_CS || a.T < 1 || a.T > moe_am_tokens(a.am) || a.am < MOE_AM_HL8 || a.am > MOE_AM_HL16)
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

bool pf_router_topk_ok(const PfRouterArgs& a) { return a.split && a.E <= 512 && a.d / 256 <= 16; }

hipError_t launch_pf_router_topk(const PfRouterArgs& a, int k, int32_t* idx, float* w, hipStream_t s) {
  if (!pf_router_topk_ok(a) || k < 1 || k > a.E) return hipErrorInvalidValue;
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + 3) / 4), block(256);
  if (a.d / 256 <= 10) hipLaunchKernelGGL(pf_router_topk_kernel<10>, grid, block, 0, s, a, k, idx, w);
  else hipLaunchKernelGGL(pf_router_topk_kernel<16>, grid, block, 0, s, a, k, idx, w);
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
