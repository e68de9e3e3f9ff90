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
//
// Memory: every wave issues the loads of all the weight chunks it will use
// before its first multiply, so each wave keeps several 128-bit loads per
// lane in flight from HBM; activation fragments come from L2.
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

// A-fragment and accumulator seed of block b; rows of tokens that do not
// exist (or are not routed here) are zero and are not loaded.
DEVI void load_a(const _Float16* frag, const float* sum, size_t b, int lane, half8_t& A, float4_t& cin) {
  A = *reinterpret_cast<const half8_t*>(frag + (b * 64 + lane) * 8);
  cin = *reinterpret_cast<const float4_t*>(sum + b * 16 + 4 * (lane >> 4));
}

// ---------------------------------------------------------------------------
// Slot list, built in LDS by a workgroup from the routing rows (T*k
// entries): routed experts are marked in a bitmap, numbered in ascending id
// order after the shared expert's slot 0, and every (token, rank) entry puts
// its gate weight in its slot's row.
// ---------------------------------------------------------------------------
struct SlotLds {
  uint32_t mark[MOE_MAX_E / 32];
  int wbase[MOE_MAX_E / 32];
  int expert[MOE_MAX_SLOTS];
  float w[MOE_MAX_SLOTS][8];
  int n_routed;
};

DEVI void build_slots(SlotLds& S, int r_e, float r_w, int tk, int k, int T, int E, bool has_shared) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nwords = (E + 31) >> 5, base = has_shared ? 1 : 0;
  for (int i = tid; i < nwords; i += blockDim.x) S.mark[i] = 0u;
  __syncthreads();
  const bool valid = tid < tk && r_e >= 0 && r_e < E;
  if (valid) atomicOr(&S.mark[r_e >> 5], 1u << (r_e & 31));
  __syncthreads();
  if (wv == 0) {
    const int c0 = (2 * lane < nwords) ? __popc(S.mark[2 * lane]) : 0;
    const int c1 = (2 * lane + 1 < nwords) ? __popc(S.mark[2 * lane + 1]) : 0;
    int incl = c0 + c1;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int excl = incl - c0 - c1;
    if (2 * lane < nwords) S.wbase[2 * lane] = excl;
    if (2 * lane + 1 < nwords) S.wbase[2 * lane + 1] = excl + c0;
    if (lane == 63) S.n_routed = incl;
  }
  __syncthreads();
  for (int i = tid; i < nwords; i += blockDim.x) {
    uint32_t m = S.mark[i];
    int slot = base + S.wbase[i];
    while (m) {
      const int bit = __builtin_ctz(m);
      S.expert[slot++] = 32 * i + bit;
      m &= m - 1u;
    }
  }
  if (has_shared && tid == 0) S.expert[0] = E;
  const int ns = base + S.n_routed;
  for (int i = tid; i < ns * 8; i += blockDim.x) S.w[i >> 3][i & 7] = (has_shared && i < 8 && i < T) ? 1.0f : 0.f;
  __syncthreads();
  if (valid) {
    const int word = r_e >> 5;
    const int slot = base + S.wbase[word] + __popc(S.mark[word] & ((1u << (r_e & 31)) - 1u));
    S.w[slot][tid / k] = r_w;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// gate/up: a work item is (slot u, group q of 64 intermediate rows = four
// 16-row tiles; the last group of an expert may have two).  The grid is
// persistent: workgroups stride over the items, the shared expert's first
// (they need no routing, so they start streaming at once), then the routed
// slots'.  Wave w of a workgroup takes k-group w (256 inputs): it issues the
// loads of its eight weight chunks (gate/up x four row tiles) into registers
// and copies its eight activation fragments and block sums straight into a
// wave-private LDS area (global_load_lds), then runs the 64 MFMAs, scaling
// each block's result as soon as it is ready.  Waves reduce through the same
// LDS area in a fixed order.  Epilogue (row tiles spread over the waves): divide by the
// token's rms (stacked layers), h = silu(g) * u, times the token's gate
// weight, written as fp16 hi/lo A-fragments (with block sums) for the down
// kernel.
// ---------------------------------------------------------------------------
constexpr int GU_MAXW = 10;                       // waves per workgroup
constexpr int GU_STAGE = 8 * 1024 + 8 * 64;       // bytes staged per wave
typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int BITS>
__global__ __launch_bounds__(640, 3) void gu_decode_kernel(GuArgs a) {
  constexpr int CB = BITS == 2 ? 1280 : 1792;
  __shared__ __attribute__((aligned(16))) unsigned char stage[GU_MAXW][GU_STAGE];
  __shared__ float bsum_lds[4][16];
  __shared__ SlotLds S;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  const int T = a.T, k = a.k, E = a.E, tk = a.T * a.k;
  const bool has_shared = a.has_shared != 0;
  const int base = has_shared ? 1 : 0;
  const int tiles_r = a.I / 16, tiles_s = has_shared ? a.Is / 16 : 0;
  const int pr = (tiles_r + 3) / 4, ps = (tiles_s + 3) / 4;
  const int n_kg = a.n_kg;
  // routing rows, fetched at once (used when the first routed item comes up)
  int r_e = -1;
  float r_w = 0.f;
  if (tid < tk) {
    r_e = a.idx[tid];
    r_w = a.w[tid];
  }
  bool built = false;
  if (blockIdx.x == 0) {
    build_slots(S, r_e, r_w, tk, k, T, E, has_shared);
    built = true;
    const int ns = base + S.n_routed;
    if (tid == 0) *a.n_slots = ns;
    for (int i = tid; i < ns; i += blockDim.x) a.slot_expert[i] = S.expert[i];
    for (int i = tid; i < ns * 8; i += blockDim.x) a.slot_w[i] = S.w[i >> 3][i & 7];
  }

  for (int item = blockIdx.x;; item += gridDim.x) {
    int u, q, ntile;
    const uint8_t* ebase;
    int64_t og, ou;
    if (item < ps) {
      u = 0;
      q = item;
      ntile = min(4, tiles_s - 4 * q);
      ebase = a.X.shared;
      og = a.X.sh_off_gate;
      ou = a.X.sh_off_up;
    } else {
      if (!built) {
        build_slots(S, r_e, r_w, tk, k, T, E, has_shared);
        built = true;
      }
      const int ri = item - ps;
      if (ri >= S.n_routed * pr) break;
      u = base + ri / pr;
      q = ri - (ri / pr) * pr;
      ntile = min(4, tiles_r - 4 * q);
      ebase = a.X.experts + (int64_t)S.expert[u] * a.X.ex_stride;
      og = a.X.off_gate;
      ou = a.X.off_up;
    }
    const uint8_t* gate = ebase + og;
    const uint8_t* up = ebase + ou;
    // epilogue operands, fetched early: the wave's tokens and their weights
    const int tok_e = 4 * ((lane >> 4) & 1);
    float rn4[4], gw4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rn4[i] = a.rnorm[tok_e + i];
      gw4[i] = (u == 0 && has_shared) ? (tok_e + i < T ? 1.0f : 0.f) : S.w[u][tok_e + i];
    }

    float4_t acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int m = 0; m < 2; ++m) acc[t][m] = float4_t{0.f, 0.f, 0.f, 0.f};

    unsigned char* st = stage[wv];
    for (int kg = wv; kg < n_kg; kg += nw) {
      ChunkRegs<BITS> c[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < ntile) {
          const int64_t ch = ((int64_t)(4 * q + t) * n_kg + kg) * CB;
          load_chunk<BITS>(c[t][0], gate + ch, lane);
          load_chunk<BITS>(c[t][1], up + ch, lane);
        }
      // activation fragments and block sums of the k-group, straight to LDS
#pragma unroll
      for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_global_load_lds(a.xfrag + (((size_t)kg * 8 + j) * 64 + lane) * 8, (lds_ptr_t)(st + 1024 * j),
                                         16, 0, 0);
      if (lane < 32)
        __builtin_amdgcn_global_load_lds(a.xsum + (size_t)kg * 8 * 16 + 4 * lane, (lds_ptr_t)(st + 8192), 16, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half8_t A = *reinterpret_cast<const half8_t*>(st + 1024 * j + 16 * lane);
        const float4_t cin = *reinterpret_cast<const float4_t*>(st + 8192 + 64 * j + 16 * (lane >> 4));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < ntile) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const float4_t C = mfma16x16x32(A, chunk_frag<BITS>(c[t][m], j), cin);
              acc[t][m] += chunk_scale(c[t][m].scales, j) * C;
            }
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // reduce the waves' partial sums in wave order (staging area reused)
    __syncthreads();
    float* red = reinterpret_cast<float*>(stage[wv]);  // [32][64]
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((t * 2 + m) * 4 + i) * 64 + lane] = acc[t][m][i];
    __syncthreads();
    for (int t = wv; t < ntile; t += nw) {  // wave wv finishes row tiles wv, wv + nw, ...
      float v[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float part[GU_MAXW];
#pragma unroll
          for (int w = 0; w < GU_MAXW; ++w)
            part[w] = reinterpret_cast<const float*>(stage[w < nw ? w : 0])[((t * 2 + m) * 4 + i) * 64 + lane];
          float sm = part[0];
#pragma unroll
          for (int w = 1; w < GU_MAXW; ++w)
            if (w < nw) sm += part[w];
          v[m][i] = add_partner32(sm);  // hi + lo parts of the token
        }
      // lane l: column n = l & 15 (intermediate row 64q + 16t + n), rows
      // m = 4(l>>4) + i, i.e. tokens tok_e + i; lanes >= 32 write the lo parts
      const int n = lane & 15;
      const bool lo_half = lane >= 32;
      const int pblk = 2 * q + (t >> 1);  // 32-row block of the down projection
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tok_e + i;
        const float g = v[0][i] / rn4[i];
        const float uu = v[1][i] / rn4[i];
        const float hv = g / (1.0f + expf(-g)) * uu;
        const float hs = (gw4[i] != 0.f) ? gw4[i] * hv : 0.f;
        const _Float16 hi = (_Float16)hs;
        const _Float16 val = lo_half ? (_Float16)(hs - (float)hi) : hi;
        const int mrow = tok + (lo_half ? 8 : 0);
        const int kk = 16 * (t & 1) + n;
        a.hfrag[(((size_t)u * a.nbI + pblk) * 64 + mrow + 16 * (kk >> 3)) * 8 + (kk & 7)] = val;
        const float sm = row16_sum((float)val);
        if (n == 0) bsum_lds[t][4 * (lane >> 4) + i] = sm;
      }
    }
    __syncthreads();
    if (tid < 16 * (ntile / 2)) {
      const int blk = tid >> 4, mr = tid & 15;
      const float sm = bsum_lds[2 * blk][mr] + bsum_lds[2 * blk + 1][mr];
      a.hsum[((size_t)u * a.nbI + 2 * q + blk) * 16 + mr] = -(float)a.code_off * sm;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// down: workgroup = (row group rg of 16*RT output rows, split s).  It sums,
// for every slot u = s, s+S, ... of the slot list, the down projection of the
// gate-weighted h, so the
// combine across experts happens in the accumulators.  Items (slot, k-group)
// go to the waves in batches of two; a batch's weight chunks and activation
// fragments are all loaded before its first multiply.  Waves reduce through
// LDS in a fixed order and the split's partial result is written to
// ypart[s]; the consumer adds the S splits in split order, so the output does
// not depend on timing.
// ---------------------------------------------------------------------------
template <int BITS, int RT>
__global__ __launch_bounds__(512) void down_decode_kernel(DownArgs a) {
  constexpr int CB = BITS == 2 ? 1280 : 1792;
  constexpr int BK = 8 / RT;
  constexpr int BATCH = 2;
  __shared__ float red[8][RT * 4][64];
  const int rg = blockIdx.x, sp = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int ns = *a.n_slots;
  const int S = a.S;
  // slots of this split: sp, sp + S, ...; slot 0 is the shared expert when
  // there is one (split 0 then starts with its k-groups)
  const bool sh_here = a.has_shared && sp == 0;
  const int first_r = sh_here ? S : sp;  // first routed slot of the split
  const int n_rs = (first_r < ns) ? (ns - first_r + S - 1) / S : 0;
  const int n_sh = sh_here ? a.n_kg_s : 0;
  const int n_items = n_sh + n_rs * a.n_kg_r;

  float4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int b0 = wv; b0 < n_items; b0 += nw * BATCH) {
    ChunkRegs<BITS> c[BATCH];
    half8_t A[BATCH][BK];
    float4_t cin[BATCH][BK];
    bool ok[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int it = b0 + q * nw;
      ok[q] = it < n_items;
      const int itc = ok[q] ? it : b0;  // keep every address valid
      int u, kg, n_kg;
      const uint8_t* mat;
      if (itc < n_sh) {
        u = 0;
        kg = itc;
        n_kg = a.n_kg_s;
        mat = a.X.shared + a.X.sh_off_down;
      } else {
        const int ri = itc - n_sh;
        u = first_r + S * (ri / a.n_kg_r);
        kg = ri % a.n_kg_r;
        n_kg = a.n_kg_r;
        mat = a.X.experts + (int64_t)a.slot_expert[u] * a.X.ex_stride + a.X.off_down;
      }
      load_chunk<BITS>(c[q], mat + ((int64_t)rg * n_kg + kg) * CB, lane);
#pragma unroll
      for (int j = 0; j < BK; ++j)
        load_a(a.hfrag, a.hsum, (size_t)u * a.nbI + kg * BK + j, lane, A[q][j], cin[q][j]);
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (!ok[q]) continue;
#pragma unroll
      for (int j = 0; j < BK; ++j)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int f = t * BK + j;
          const float4_t C = mfma16x16x32(A[q][j], chunk_frag<BITS>(c[q], f), cin[q][j]);
          acc[t] += chunk_scale(c[q].scales, f) * C;
        }
    }
  }

#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][t * 4 + i][lane] = acc[t][i];
  __syncthreads();
  if (wv != 0) return;
  const int T = a.T, d = a.d, n = lane & 15;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float part[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) part[w] = red[w < nw ? w : 0][t * 4 + i][lane];
      float s = part[0];
#pragma unroll
      for (int w = 1; w < 8; ++w)
        if (w < nw) s += part[w];
      s = add_partner32(s);
      const int tok = 4 * (lane >> 4) + i;  // lanes < 32 hold tokens 0..7
      const int o = rg * 16 * RT + 16 * t + n;
      if (lane < 32 && tok < T) a.ypart[((size_t)sp * 8 + tok) * d + o] = s;
    }
}

template <int BITS, int RT>
hipError_t launch_down_t(const DownArgs& a, int grid_x, int nw, hipStream_t s) {
  hipLaunchKernelGGL((down_decode_kernel<BITS, RT>), dim3(grid_x, a.S), dim3(64 * nw), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gu_decode(const GuArgs& a, int n_wg, hipStream_t s) {
  int nw = a.n_kg < 10 ? a.n_kg : 10;
  if (a.bits == 2) hipLaunchKernelGGL(gu_decode_kernel<2>, dim3(n_wg), dim3(64 * nw), 0, s, a);
  else hipLaunchKernelGGL(gu_decode_kernel<3>, dim3(n_wg), dim3(64 * nw), 0, s, a);
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
