// prefill.hip -- chunked prefill (T > 8 tokens per call): the layer for a
// prompt chunk of up to thousands of tokens [agentlenshq article, section
// "Strata 如何让 125 B 模型适配 12-24 GB 显存", last item; cnyes profile,
// section "速度倍增器"].
//
// Steps (kernels in launch order):
//   prep      per token row: power-of-two exponent ex with 2^14 <= max|x| *
//             2^-ex < 2^15, then x * 2^-ex split into fp16 hi + lo (the
//             scaling is exact and keeps every row in fp16 range);
//   router    logits = 2^(ex+ew) * (xh.wh + xh.wl + xl.wh) + bias on the
//             matrix cores (three fp16 products, ~22-bit operands, fp32
//             accumulation), then the shared top-k kernel;
//   group     token-to-expert counting sort: per 64-token tile a bitmap of
//             the tokens of each expert, a scan over tiles and experts, and a
//             permute that places pair (t, r) at row offsets[e] + (tokens of
//             e in earlier tiles) + (tokens of e earlier in its tile); rows of
//             one expert are padded to a multiple of 16 and cut into work
//             items of up to 128 rows; the shared expert's rows follow;
//   gate_up   per item and 128 intermediate columns: G = X W_g^T, U = X W_u^T
//             with the weights dequantized in registers to fp16 s * c (exact
//             for 2-bit codes, one rounding for 3-bit), x rows gathered
//             into LDS by direct-to-LDS loads, v_mfma_f32_16x16x32_f16;
//             epilogue h = silu(g) * u in fp32, stored as fp16(h 2^-eh)
//             with eh = hb + 2 ex: hb is a per-expert bound exponent found at
//             pack time from the row L1 norms of gate and up, so no pass over
//             the row is needed to choose it;
//   down      per item and 256 output columns: Y = H W_d^T with H staged into
//             LDS by direct-to-LDS loads; the epilogue writes one fp16 row
//             per pair, fp16(sum 2^-ed) with ed a per-expert pack-time bound,
//             and the row's factor w 2^(eh + ed);
//   combine   y[t] = sum of its pairs' factor times row in rank order + its
//             shared row.
// Every product on the matrix cores is exact; the roundings are the fp16
// activations (x, h), 3-bit weights with a code of +-3, the fp16 down rows,
// and fp32 accumulation.
#include <type_traits>

#include "kern_common.h"
#include "moe_launch.h"

namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void* lds_ptr_t;

DEVI _Float16 half_of_bits(uint32_t b) {
  _Float16 h;
  const uint16_t v = (uint16_t)b;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

// ---------------------------------------------------------------------------
// Weight registers of one 16-row tile for up to 8 fragments (a full chunk) or
// 4 fragments (half a chunk: codes and scales in elements [0..1], high bits
// in hi[0]).  Fragment f: codes dword f/2 at shift 2(f%2), fp16 scale half f,
// high bits dword f/4 at bit f%4.  Codebook blocks (MOE_KIND_CB): codes hold
// the index low bytes (bytes 2f, 2f+1), hi the sign bits (byte f), ih the
// index high bits (bits 2f, 2f+1), all renumbered from the half's first
// fragment for a half chunk.
// ---------------------------------------------------------------------------
struct WRegs {
  u32x4_t codes;
  u32x4_t scales;
  u32x2_t hi;
  uint32_t ih;
};

template <int BITS>
DEVI void load_full(WRegs& w, const uint8_t* chunk, int lane) {
  w.codes = ld128(chunk + 16 * lane);
  w.scales = ld128(chunk + 1024 + 16 * (lane & 15));
  if constexpr (BITS != 2) w.hi = ld64(chunk + 1280 + 8 * lane);
  if constexpr (BITS == MOE_KIND_CB) w.ih = *reinterpret_cast<const uint16_t*>(chunk + 1792 + 2 * lane);
}

// fragments 4h..4h+3 of a chunk
template <int BITS>
DEVI void load_half(WRegs& w, const uint8_t* chunk, int h, int lane) {
  const u32x2_t c = ld64(chunk + 16 * lane + 8 * h);
  const u32x2_t s = ld64(chunk + 1024 + 16 * (lane & 15) + 8 * h);
  w.codes = u32x4_t{c[0], c[1], 0u, 0u};
  w.scales = u32x4_t{s[0], s[1], 0u, 0u};
  if constexpr (BITS != 2) w.hi = u32x2_t{*reinterpret_cast<const uint32_t*>(chunk + 1280 + 8 * lane + 4 * h), 0u};
  if constexpr (BITS == MOE_KIND_CB) w.ih = (uint32_t)chunk[1792 + 2 * lane + h];
}

// w = s * (q - 2^(b-1)) for the lane's 8 codes of fragment f, in fp16: q is
// exact from the fp4 conversion, the fused multiply-add rounds once.
// Codebook blocks: w = s * c with c the signed code from the LDS grid, one
// rounding.
template <int BITS>
DEVI half8_t dequant(const WRegs& w, int f) {
  const uint32_t sd = w.scales[f >> 1];
  const _Float16 s = half_of_bits((f & 1) ? (sd >> 16) : sd);
  const half8_t sv = s;
  if constexpr (BITS == MOE_KIND_CB) {
    return frag_cb(w.codes, w.ih, w.hi, f, cb_grid_lds) * sv;
  } else {
    const uint32_t dw = w.codes[f >> 1];
    half8_t q = nibbles_to_half8(((f & 1) ? (dw >> 2) : dw) & 0x33333333u, 2.0f);
    if constexpr (BITS == 3) q += nibbles_to_half8((w.hi[f >> 2] >> (f & 3)) & 0x11111111u, 8.0f);
    const half8_t ov = sv * (_Float16)(-(float)(1 << (BITS - 1)));
    return __builtin_elementwise_fma(q, sv, ov);
  }
}

// ---------------------------------------------------------------------------
// Router weights, prepared at pack time: row exponent ew (as for x) and the
// row times 2^-ew split into fp16 hi + lo, stored as MFMA B fragments
// [E16/16][d/32][64 lanes][8]: lane l holds row 16*tile + l%16, inputs
// 32*block + 8*(l/16) .. +8.  Rows E..E16-1 are zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_router_kernel(const float* W, int E, int E16, int d, _Float16* wh,
                                                          _Float16* wl, int32_t* ew) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wv;
  if (e >= E16) return;
  const bool valid = e < E;
  const float* row = W + (size_t)(valid ? e : 0) * d;
  float m = 0.f;
  if (valid)
    for (int c = 4 * lane; c < d; c += 256) {
      const float4_t v = *reinterpret_cast<const float4_t*>(row + c);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
  m = wave_max(m);
  const int x = fp16_exponent_for(m);
  if (lane == 0) ew[e] = x;
  const int nb = d / 32;
  for (int g = lane; g < d / 8; g += 64) {
    half8_t hi, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = valid ? ldexpf(row[8 * g + i], -x) : 0.f;
      const _Float16 h = (_Float16)v;
      hi[i] = h;
      lo[i] = (_Float16)(v - (float)h);
    }
    const size_t off = (((size_t)(e >> 4) * nb + (g >> 2)) * 64 + (e & 15) + 16 * (g & 3)) * 8;
    *reinterpret_cast<half8_t*>(wh + off) = hi;
    *reinterpret_cast<half8_t*>(wl + off) = lo;
  }
}

// ---------------------------------------------------------------------------
// Exponent bases of one expert, prepared at pack time.  Lg = max over gate
// rows of sum_j |w_ij|, Lu likewise for up, Ld for down.  For an input row
// scaled to |x_j| < 2^15 (x times 2^-ex), |g| <= Lg 2^(15 + ex),
// |u| <= Lu 2^(15 + ex) and |silu(g) u| <= |g| |u|, so with 2^e > Lg Lu the
// value h 2^-(hb + 2 ex) with hb = e + 16 is below 2^14 (2^15 allowing for
// the fp32 rounding of the sums): the fp16 intermediate needs no pass over
// the row to choose its exponent.  The down sums over such fp16 values are
// below 2^15 Ld, so with 2^ed > Ld they are stored as fp16(sum 2^-ed), below
// 2^15.  One workgroup per expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_hbound_kernel(const uint8_t* canon, int64_t stride, int I, int d, int bits,
                                                          const uint8_t* grid, int32_t* hb, int32_t* ed) {
  __shared__ float red[3][4];
  const uint8_t* ex = canon + (int64_t)blockIdx.x * stride;
  const bool cbk = bits == MOE_KIND_CB;
  const int nb = d / 32, nbI = I / 32, bb = cbk ? 15 : 2 + 4 * bits, off = cbk ? 0 : 1 << (bits - 1);
  float lmax[3] = {0.f, 0.f, 0.f};
  for (int m = 0; m < 3; ++m) {
    const uint8_t* mat = ex + (int64_t)m * I * nb * bb;
    const int nrow = m < 2 ? I : d, nblk = m < 2 ? nb : nbI;
    for (int i = threadIdx.x; i < nrow; i += 256) {
      float sum = 0.f;
      for (int b = 0; b < nblk; ++b) {
        const uint8_t* B = mat + ((int64_t)i * nblk + b) * bb;
        const float sc = fabsf(half_bits_to_float((uint32_t)B[0] | ((uint32_t)B[1] << 8)));
        int cs = 0;
        if (cbk) {
          // the magnitudes of the block's eight grid entries (signs do not count)
          for (int i = 0; i < 8; ++i) {
            const int index = B[2 + i] | (((B[10] >> i) & 1) << 8);
            for (int c = 0; c < 4; ++c) cs += grid[4 * index + c];
          }
        } else {
          for (int j = 0; j < 32; ++j) {
            const int bit = bits * j, by = bit >> 3;
            const uint32_t v = (uint32_t)B[2 + by] | (by + 1 < 4 * bits ? (uint32_t)B[3 + by] << 8 : 0u);
            cs += abs((int)((v >> (bit & 7)) & ((1u << bits) - 1u)) - off);
          }
        }
        sum += sc * (float)cs;
      }
      lmax[m] = fmaxf(lmax[m], sum);
    }
  }
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int m = 0; m < 3; ++m) {
    const float v = wave_max(lmax[m]);
    if (lane == 0) red[m][wv] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float l[3];
    for (int m = 0; m < 3; ++m) l[m] = fmaxf(fmaxf(red[m][0], red[m][1]), fmaxf(red[m][2], red[m][3]));
    const float p = l[0] * l[1];
    int e = 0;
    if (p > 0.f) frexpf(p, &e);  // p < 2^e
    hb[blockIdx.x] = e + 16;
    int e2 = 0;
    if (l[2] > 0.f) frexpf(l[2], &e2);  // Ld < 2^e2
    ed[blockIdx.x] = e2;
  }
}

// ---------------------------------------------------------------------------
// prep: one wave per token row.  With norm set the row is first divided by
// sqrt(mean(x^2) + eps) (the RMSNorm between stacked layers).
// ---------------------------------------------------------------------------
// One row per wavefront.  Rows up to 4096 wide are loaded once into
// registers (every load in flight at once); wider rows are read twice.
template <bool RESIDENT>
DEVI void prep_row(const PfPrepArgs& a, int t, int lane) {
  constexpr int NV = 16;  // float4 per lane when resident: 4096 columns
  const float* xr = a.x + (size_t)t * a.d;
  float4_t v[RESIDENT ? NV : 1];
  float m = 0.f, ss = 0.f;
  auto acc = [&](const float4_t& u) {
    m = fmaxf(m, fmaxf(fmaxf(fabsf(u[0]), fabsf(u[1])), fmaxf(fabsf(u[2]), fabsf(u[3]))));
    ss = fmaf(u[0], u[0], ss);
    ss = fmaf(u[1], u[1], ss);
    ss = fmaf(u[2], u[2], ss);
    ss = fmaf(u[3], u[3], ss);
  };
  if constexpr (RESIDENT) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      v[i] = *reinterpret_cast<const float4_t*>(xr + min(4 * lane + 256 * i, a.d - 4));  // clamped; unused past d
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (4 * lane + 256 * i < a.d) acc(v[i]);
  } else {
    for (int c = 4 * lane; c < a.d; c += 256) acc(*reinterpret_cast<const float4_t*>(xr + c));
  }
  m = wave_max(m);
  float rms = 1.f;
  if (a.norm) {
    ss = wave_sum(ss);
    rms = sqrtf(ss / (float)a.d + a.eps);
    m = m / rms;  // division is monotonic: the largest quotient is the quotient of the largest
  }
  const int ex = fp16_exponent_for(m);
  if (lane == 0) a.ex[t] = ex;
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  auto put = [&](const float4_t& u, int c) {
    h4_t h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = ldexpf(a.norm ? u[i] / rms : u[i], -ex);
      h[i] = (_Float16)s;
      l[i] = (_Float16)(s - (float)h[i]);
    }
    *reinterpret_cast<h4_t*>(a.xh + (size_t)t * a.d + c) = h;
    *reinterpret_cast<h4_t*>(a.xl + (size_t)t * a.d + c) = l;
  };
  if constexpr (RESIDENT) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (4 * lane + 256 * i < a.d) put(v[i], 4 * lane + 256 * i);
  } else {
    for (int c = 4 * lane; c < a.d; c += 256) put(*reinterpret_cast<const float4_t*>(xr + c), c);
  }
}

__global__ __launch_bounds__(256) void pf_prep_kernel(PfPrepArgs a) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wv;
  if (t >= a.T) return;
  if (a.d <= 4096) prep_row<true>(a, t, lane);
  else prep_row<false>(a, t, lane);
}

template <int P>
using ic = std::integral_constant<int, P>;

// s_waitcnt immediate (gfx9 encoding): wait until at most n vector-memory
// operations of this wave are outstanding; LDS and export counters free.
constexpr int16_t vmcnt_imm(int n) { return (int16_t)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8)); }

// Pipeline stages in separate LDS arrays, so that the compiler can see that
// a direct-to-LDS load into one stage does not alias reads of another (with
// one array it waits for every outstanding load before each LDS read).  The
// router GEMM uses three (step s in stage s % 3, loads two steps ahead), the
// grouped GEMMs two (step s in stage s % 2, loads one step ahead, two
// workgroups per CU).
struct Stages {
  unsigned char* s0;
  unsigned char* s1;
  unsigned char* s2;
  template <int P>
  DEVI unsigned char* get() const { return P == 0 ? s0 : P == 1 ? s1 : s2; }
};

// ---------------------------------------------------------------------------
// router GEMM: workgroup = 128 tokens x 128 experts, wave = 128 tokens x 32
// experts; x hi/lo fragments staged in LDS by direct loads (2 blocks per
// step, three stages), weight fragments straight into registers.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void pf_router_kernel(PfRouterArgs a) {
  constexpr int KS = 2;
  constexpr int STAGE = 2 * 8 * KS * 1024;  // [hi/lo][row group][block] fragments
  __shared__ __attribute__((aligned(1024))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[STAGE];
  const Stages S{st0, st1, st2};
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int row0 = blockIdx.x * 128;
  const int nb = a.d / 32, n_et = a.E16 / 16;
  // eight wavefronts (two per SIMD), one 16-expert tile each
  constexpr int NJ = 1;
  const int et0 = blockIdx.y * 8 + wv;
  const bool act0 = et0 < n_et, act1 = false;
  const int etl[NJ] = {act0 ? et0 : 0};  // an idle wave loads (and ignores) tile 0
  int tok[8];
#pragma unroll
  for (int rg = 0; rg < 8; ++rg) tok[rg] = min(row0 + 16 * rg + n, a.T - 1);
  // this wave stages part hl (hi or lo) of block dkb of row groups 4 rh .. 4 rh + 3
  const int hl = (wv >> 1) & 1, dkb = wv & 1, rh = wv >> 2;
  const _Float16* asrc = hl ? a.xl : a.xh;

  // acc: the current 256-column slice (4 steps) from zero; tot: the slices
  // added in order, so a split launch (one slice per workgroup, added by the
  // reduce kernel in the same order) gives the same bits
  float4_t acc[8][NJ], tot[8][NJ];
#pragma unroll
  for (int rg = 0; rg < 8; ++rg)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[rg][j] = tot[rg][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int LOADS = 4 + KS * NJ * 2;
  static_assert(256 / 32 == 4 * KS, "a slice is four steps");
  u32x4_t bh[3][KS][NJ], bl[3][KS][NJ];
  const int sbase = a.split ? 4 * blockIdx.z : 0;  // first step of this workgroup
  const int nsteps = a.split ? 4 : nb / KS;
  auto issue = [&](auto P_, int ls) {
    constexpr int P = decltype(P_)::value;
    const int s = sbase + ls;
    unsigned char* st = S.get<P>();
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int rg = 4 * rh + r4;
      __builtin_amdgcn_global_load_lds(asrc + (size_t)tok[rg] * a.d + (KS * s + dkb) * 32 + 8 * q,
                                       (lds_ptr_t)(st + ((hl * 8 + rg) * KS + dkb) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < KS; ++kb)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const size_t off = (((size_t)etl[j] * nb + KS * s + kb) * 64 + lane) * 8;
        bh[P][kb][j] = ld128(a.wh + off);
        bl[P][kb][j] = ld128(a.wl + off);
      }
  };
  auto step = [&](auto P_, int s) {  // s: step of this workgroup
    constexpr int P = decltype(P_)::value;
    if (s + 1 < nsteps) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (s + 2 < nsteps) issue(ic<(P + 2) % 3>{}, s + 2);
    if (act0) {
      const unsigned char* st = S.get<P>();
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) {
        half8_t ah[8], al[8];
#pragma unroll
        for (int rg = 0; rg < 8; ++rg) {
          ah[rg] = *reinterpret_cast<const half8_t*>(st + ((0 * 8 + rg) * KS + kb) * 1024 + 16 * lane);
          al[rg] = *reinterpret_cast<const half8_t*>(st + ((1 * 8 + rg) * KS + kb) * 1024 + 16 * lane);
        }
#pragma unroll
        for (int term = 0; term < 3; ++term)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if (j == 0 || act1) {
              const half8_t B = __builtin_bit_cast(half8_t, term == 1 ? bl[P][kb][j] : bh[P][kb][j]);
#pragma unroll
              for (int rg = 0; rg < 8; ++rg) acc[rg][j] = mfma16x16x32(term == 2 ? al[rg] : ah[rg], B, acc[rg][j]);
            }
      }
    }
    if ((s & 3) == 3) {  // end of a slice
#pragma unroll
      for (int rg = 0; rg < 8; ++rg)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          tot[rg][j] += acc[rg][j];
          acc[rg][j] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
  };
  issue(ic<0>{}, 0);
  if (nsteps > 1) issue(ic<1>{}, 1);
  for (int s = 0; s < nsteps; s += 3) {
    step(ic<0>{}, s);
    if (s + 1 < nsteps) step(ic<1>{}, s + 1);
    if (s + 2 < nsteps) step(ic<2>{}, s + 2);
  }
#pragma unroll
  for (int rg = 0; rg < 8; ++rg)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = (et0 + j) * 16 + n;
      if (!(j == 0 ? act0 : act1) || e >= a.E) continue;
      if (a.split) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = row0 + 16 * rg + 4 * q + i;
          if (t < a.T) a.part[((size_t)blockIdx.z * a.T + t) * a.E + e] = tot[rg][j][i];
        }
        continue;
      }
      const int ewe = a.ew[e];
      const float b = a.bias[e];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = row0 + 16 * rg + 4 * q + i;
        if (t < a.T) a.logits[(size_t)t * a.E + e] = ldexpf(tot[rg][j][i], a.ex[t] + ewe) + b;
      }
    }
}

// The slices of a split router launch added in slice order from zero (the
// order the unsplit kernel uses), then scaled and biased.
__global__ __launch_bounds__(256) void pf_router_reduce_kernel(PfRouterArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * a.E) return;
  const int t = (int)(i / a.E), e = (int)(i - (int64_t)t * a.E);
  const int ns = a.d / 256;
  float tot = 0.f;
  for (int z = 0; z < ns; ++z) tot += a.part[((size_t)z * a.T + t) * a.E + e];
  a.logits[i] = ldexpf(tot, a.ex[t] + a.ew[e]) + a.bias[e];
}

// ---------------------------------------------------------------------------
// grouping (token-to-expert counting sort)
// ---------------------------------------------------------------------------
// hist: one wave per 64-token tile; bit (t mod 64) of bm[e] is set when token
// t names expert e (a repeated id of one token sets the same bit again).
__global__ __launch_bounds__(64) void pf_hist_kernel(PfGroupArgs a) {
  __shared__ unsigned long long bm[MOE_MAX_E];
  const int lane = threadIdx.x, tile = blockIdx.x;
  for (int e = lane; e < a.E; e += 64) bm[e] = 0ull;
  __syncthreads();
  const int t = tile * PF_T64 + lane;
  if (t < a.T)
    for (int r = 0; r < a.k; ++r) {
      const int e = a.idx[(size_t)t * a.k + r];
      if (e >= 0 && e < a.E) atomicOr(&bm[e], 1ull << lane);
    }
  __syncthreads();
  for (int e = lane; e < a.E; e += 64) {
    const unsigned long long v = bm[e];
    a.tile_bm[(size_t)tile * a.E + e] = v;
    a.tile_cnt[(size_t)tile * a.E + e] = __popcll(v);
  }
}

// Exclusive prefix sum over the 1024 threads of the block.
DEVI int block_exclusive_scan(int v, int* sbuf, int tid, int* total) {
  sbuf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int o = tid >= off ? sbuf[tid - off] : 0;
    __syncthreads();
    sbuf[tid] += o;
    __syncthreads();
  }
  const int incl = sbuf[tid];
  *total = sbuf[1023];
  __syncthreads();
  return incl - v;
}

// scan: one block of 1024 threads.  Per expert: counts over tiles (and the
// exclusive prefix over tiles, in place); then padded row offsets, padding
// rows, shared rows and the work-item list.
__global__ __launch_bounds__(1024) void pf_scan_kernel(PfGroupArgs a) {
  __shared__ int cnt[MOE_MAX_E];
  __shared__ int sbuf[1024];
  const int tid = threadIdx.x;
  const int E = a.E;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    int* col = a.tile_cnt + e;
    // 32 loads in flight per round trip
    for (int t0 = 0; t0 < a.n_tiles; t0 += 32) {
      int c[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) c[u] = t0 + u < a.n_tiles ? col[(size_t)(t0 + u) * E] : 0;
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (t0 + u < a.n_tiles) { col[(size_t)(t0 + u) * E] = run; run += c[u]; }
    }
    cnt[e] = run;
    a.counts[e] = run;
  }
  __syncthreads();
  // thread tid owns experts 4 tid .. 4 tid + 3
  int pc[4], ni[4], rsum = 0, isum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * tid + u;
    const int c = e < E ? cnt[e] : 0;
    pc[u] = (c + a.pad - 1) / a.pad * a.pad;
    ni[u] = (pc[u] + a.TM - 1) / a.TM;
    rsum += pc[u];
    isum += ni[u];
  }
  int rows_routed, items_routed;
  int roff = block_exclusive_scan(rsum, sbuf, tid, &rows_routed);
  int ioff = block_exclusive_scan(isum, sbuf, tid, &items_routed);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * tid + u;
    if (e < E) {
      a.offsets[e] = roff;
      for (int p = roff + cnt[e]; p < roff + pc[u]; ++p) {
        a.row_src[p] = -1;
        if (a.row_tok) { a.row_tok[p] = 0; a.row_w[p] = 0.f; }
      }
      if (a.n_items)
        for (int j = 0; j < ni[u]; ++j) {
          a.item_group[ioff + j] = e;
          a.item_row0[ioff + j] = roff + j * a.TM;
          a.item_rows[ioff + j] = min(a.TM, pc[u] - j * a.TM);
        }
    }
    roff += pc[u];
    ioff += ni[u];
  }
  const int rows_sh = a.has_shared ? (a.T + 15) / 16 * 16 : 0;
  const int items_sh = (rows_sh + a.TM - 1) / a.TM;
  if (tid == 0) {
    a.offsets[E] = rows_routed;
    if (a.n_items) {
      a.offsets[E + 1] = rows_routed + rows_sh;
      *a.n_items = items_routed + items_sh;
    }
  }
  for (int t = tid; t < rows_sh; t += 1024) {
    const int p = rows_routed + t;
    a.row_src[p] = -1;
    a.row_tok[p] = t < a.T ? t : 0;
    a.row_w[p] = t < a.T ? 1.f : 0.f;
  }
  if (a.n_items)
    for (int j = tid; j < items_sh; j += 1024) {
      a.item_group[items_routed + j] = E;
      a.item_row0[items_routed + j] = rows_routed + j * a.TM;
      a.item_rows[items_routed + j] = min(a.TM, rows_sh - j * a.TM);
    }
  for (int p = rows_routed + tid; p < a.R_fill; p += 1024) a.row_src[p] = -1;
}

// permute: one thread per (t, r).  A pair is used unless its id is outside
// [0, E) or repeats an earlier slot of the same token.
__global__ __launch_bounds__(256) void pf_permute_kernel(PfGroupArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.T * a.k) return;
  const int t = (int)(i / a.k), r = (int)(i - (int64_t)t * a.k);
  const int e = a.idx[i];
  bool ok = e >= 0 && e < a.E;
  for (int u = 0; u < r && ok; ++u) ok = a.idx[(size_t)t * a.k + u] != e;
  if (!ok) {
    if (a.slot_pos) a.slot_pos[i] = -1;
    return;
  }
  const int tile = t / PF_T64, bit = t % PF_T64;
  const size_t te = (size_t)tile * a.E + e;
  const int rank = __popcll(a.tile_bm[te] & ((1ull << bit) - 1ull));
  const int p = a.offsets[e] + a.tile_cnt[te] + rank;
  a.row_src[p] = (int32_t)i;
  if (a.row_tok) {
    a.row_tok[p] = t;
    a.row_w[p] = a.w ? a.w[i] : 1.f;
  }
  if (a.slot_pos) a.slot_pos[i] = p;
}

// Short chunks (at most PF_SMALL_T tokens, PF_SMALL_E experts and MOE_MAX_K
// ranks): the work of the three kernels above in one workgroup of 1024
// threads, with the same results (short chunks pay mostly the fixed costs of
// the layer's kernels).
// The token bitmaps of every expert per 64-token tile stay in LDS; thread e
// takes expert e's count, padded rows and work items, and the row offsets
// and item positions come from a scan over the threads in expert order (a
// lane scan per wavefront, then the sixteen wavefront totals); a pair's row
// is offsets[e] + the tokens of e in earlier tiles + its rank in its tile.
constexpr int PF_SMALL_T = 256, PF_SMALL_E = 1024;
__global__ __launch_bounds__(1024) void pf_group_small_kernel(PfGroupArgs a) {
  constexpr int PP = PF_SMALL_T * MOE_MAX_K / 1024;  // pairs per thread
  __shared__ unsigned long long bm[PF_SMALL_T / PF_T64][PF_SMALL_E];
  __shared__ int off_lds[PF_SMALL_E];
  __shared__ int ids[PF_SMALL_T * MOE_MAX_K];
  __shared__ int wsum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E, T = a.T, k = a.k, n_tiles = (T + PF_T64 - 1) / PF_T64;
  const int n_pairs = T * k;
  // the ids (and gate weights) of this thread's pairs i = tid + 1024 j are
  // loaded first and kept in registers; their loads overlap the clearing
  int myid[PP];
  float myw[PP];
#pragma unroll
  for (int j = 0; j < PP; ++j) {
    const int i = min(tid + 1024 * j, max(n_pairs - 1, 0));
    myid[j] = a.idx[i];
    myw[j] = a.w ? a.w[i] : 1.f;
  }
  for (int i = tid; i < n_tiles * PF_SMALL_E; i += 1024) bm[i / PF_SMALL_E][i % PF_SMALL_E] = 0ull;
#pragma unroll
  for (int j = 0; j < PP; ++j)
    if (tid + 1024 * j < n_pairs) ids[tid + 1024 * j] = myid[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PP; ++j) {
    const int i = tid + 1024 * j, t = i / k, e = myid[j];
    if (i < n_pairs && e >= 0 && e < E) atomicOr(&bm[t / PF_T64][e], 1ull << (t % PF_T64));
  }
  __syncthreads();
  const int e = tid;
  int cnt = 0;
  if (e < E)
    for (int j = 0; j < n_tiles; ++j) cnt += __popcll(bm[j][e]);
  const int pc = (cnt + a.pad - 1) / a.pad * a.pad;
  const int ni = (pc + a.TM - 1) / a.TM;
  int rs = pc, is = ni;  // inclusive scans within the wavefront
  for (int o = 1; o < 64; o <<= 1) {
    const int r2 = __shfl_up(rs, o, 64), i2 = __shfl_up(is, o, 64);
    if (lane >= o) {
      rs += r2;
      is += i2;
    }
  }
  if (lane == 63) {
    wsum[0][wv] = rs;
    wsum[1][wv] = is;
  }
  __syncthreads();
  int rows_routed = 0, items_routed = 0, rb = 0, ib = 0;
  for (int w = 0; w < 16; ++w) {
    const int r = wsum[0][w], it = wsum[1][w];
    if (w < wv) {
      rb += r;
      ib += it;
    }
    rows_routed += r;
    items_routed += it;
  }
  const int roff = rb + rs - pc, ioff = ib + is - ni;
  if (e < E) {
    a.counts[e] = cnt;
    a.offsets[e] = roff;
    off_lds[e] = roff;
    for (int p = roff + cnt; p < roff + pc; ++p) {
      a.row_src[p] = -1;
      if (a.row_tok) { a.row_tok[p] = 0; a.row_w[p] = 0.f; }
    }
    if (a.n_items)
      for (int j = 0; j < ni; ++j) {
        a.item_group[ioff + j] = e;
        a.item_row0[ioff + j] = roff + j * a.TM;
        a.item_rows[ioff + j] = min(a.TM, pc - j * a.TM);
      }
  }
  const int rows_sh = a.has_shared ? (T + 15) / 16 * 16 : 0;
  const int items_sh = (rows_sh + a.TM - 1) / a.TM;
  if (tid == 0) {
    a.offsets[E] = rows_routed;
    if (a.n_items) {
      a.offsets[E + 1] = rows_routed + rows_sh;
      *a.n_items = items_routed + items_sh;
    }
  }
  for (int t = tid; t < rows_sh; t += 1024) {
    const int p = rows_routed + t;
    a.row_src[p] = -1;
    a.row_tok[p] = t < T ? t : 0;
    a.row_w[p] = t < T ? 1.f : 0.f;
  }
  if (a.n_items)
    for (int j = tid; j < items_sh; j += 1024) {
      a.item_group[items_routed + j] = E;
      a.item_row0[items_routed + j] = rows_routed + j * a.TM;
      a.item_rows[items_routed + j] = min(a.TM, rows_sh - j * a.TM);
    }
  for (int p = rows_routed + tid; p < a.R_fill; p += 1024) a.row_src[p] = -1;
  __syncthreads();  // every expert's offset in LDS
  // a pair is used unless its id is outside [0, E) or repeats an earlier
  // slot of the same token
#pragma unroll
  for (int j = 0; j < PP; ++j) {
    const int i = tid + 1024 * j;
    if (i >= n_pairs) break;
    const int t = i / k, r = i - t * k, ei = myid[j];
    bool ok = ei >= 0 && ei < E;
    for (int u = 0; u < r && ok; ++u) ok = ids[t * k + u] != ei;
    if (!ok) {
      if (a.slot_pos) a.slot_pos[i] = -1;
      continue;
    }
    const int tile = t / PF_T64, bit = t % PF_T64;
    int p = off_lds[ei] + __popcll(bm[tile][ei] & ((1ull << bit) - 1ull));
    for (int j = 0; j < tile; ++j) p += __popcll(bm[j][ei]);
    a.row_src[p] = i;
    if (a.row_tok) {
      a.row_tok[p] = t;
      a.row_w[p] = myw[j];
    }
    if (a.slot_pos) a.slot_pos[i] = p;
  }
}

// ---------------------------------------------------------------------------
// gate/up grouped GEMM.  Workgroup: one work item (up to 128 rows of one
// expert) x 128 intermediate columns; wave wv: all rows x columns
// h0 = 128 nt + 32 wv .. +32 of both gate and up (4 tiles of 16 weight rows).
// Per step of 4 blocks (128 inputs): A fragments [row group][block] in LDS
// (wave wv stages block wv of every row group), weights of the step (half
// a chunk per tile) in registers, double buffered.
// ---------------------------------------------------------------------------
constexpr int GEMM_STAGE = 8 * 4 * 1024;  // [row group][block] fragments of one step

// Work-item placement.  Workgroups are dispatched to the 8 XCDs (each with its
// own L2) in turn: workgroup b runs on XCD b % 8.  XCD x takes the x-th
// contiguous eighth of the item list, and the n_nt column tiles of one item
// run back to back on it, so an item's activation rows and an expert's
// weights are fetched into one L2 and reused there.  The grid has
// 8 * ceil(max_items / 8) * n_nt workgroups; the surplus exits at once.
constexpr int N_XCD = 8;
DEVI bool xcd_tile(int n_items, int n_nt, int* item, int* nt) {
  const int x = blockIdx.x % N_XCD, j = blockIdx.x / N_XCD;
  const int ipx = (n_items + N_XCD - 1) / N_XCD;
  const int li = j / n_nt;
  *item = x * ipx + li;
  *nt = j - li * n_nt;
  return li < ipx && *item < n_items;
}

template <int BITS, int NRG>
DEVI void gate_up_item(const PfGemmArgs& a, const Stages& S, int* ex_lds, int g, int row0, int rows, int nt) {
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 15, q = lane >> 4;
  const bool shared = g == a.E;
  const int Ig = shared ? a.Is : a.I;
  const uint8_t* eb = shared ? a.X.shared : a.X.experts + (int64_t)g * a.X.ex_stride;
  const int h0 = nt * PF_HT + 32 * wv;
  const bool act = h0 < Ig;
  const int nkg = a.d / 256;
  constexpr int CB = moe_chunk_bytes(BITS);
  const uint8_t* cp[4];
  {
    const uint8_t* gate = eb + (shared ? a.X.sh_off_gate : a.X.off_gate);
    const uint8_t* up = eb + (shared ? a.X.sh_off_up : a.X.off_up);
    const int hr = act ? h0 : 0;  // idle waves load (and ignore) row group 0
    cp[0] = gate + (int64_t)(hr / 16) * nkg * CB;
    cp[1] = cp[0] + (int64_t)nkg * CB;
    cp[2] = up + (int64_t)(hr / 16) * nkg * CB;
    cp[3] = cp[2] + (int64_t)nkg * CB;
  }
  // A staging: a stage holds the step's 128 inputs of every row, 256 B per
  // row, its sixteen 16-byte slots swizzled (slot s of row r holds input
  // slot s ^ (r & 15)) so that the MFMA reads below hit distinct banks.
  // One direct-to-LDS load fills 4 whole rows (two full cache lines each);
  // wave wv issues loads wv, wv + 4, ... (rows 4 (wv + 4 i) + lane / 16).
  const int lrow = lane >> 4;
  const int gslot = (lane & 15) ^ (((4 * wv + lrow) & 15));  // same for every i: 16 i leaves r & 15 unchanged
  const _Float16* arow[NRG];
#pragma unroll
  for (int i = 0; i < NRG; ++i) {
    const int r = 4 * (wv + 4 * i) + lrow;
    arow[i] = a.xh + (size_t)(r < rows ? a.row_tok[row0 + r] : 0) * a.d + 8 * gslot;
  }
  if (tid < PF_TM) ex_lds[tid] = a.ex[tid < rows ? a.row_tok[row0 + tid] : 0];
  int xs[4];  // swizzled byte offset of the lane's A slot for each block of a step
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) xs[kb] = n * 256 + (((4 * kb + q) ^ n) << 4);

  float4_t acc[NRG][4];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[rg][m] = float4_t{0.f, 0.f, 0.f, 0.f};

  WRegs bw[2][4];
  const int nsteps = a.d / 128;
  auto issue = [&](auto P_, int s) {
    constexpr int P = decltype(P_)::value;
    unsigned char* st = S.get<P>();
#pragma unroll
    for (int i = 0; i < NRG; ++i)
      __builtin_amdgcn_global_load_lds(arow[i] + 128 * s, (lds_ptr_t)(st + (wv + 4 * i) * 1024), 16, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) load_half<BITS>(bw[P][m], cp[m] + (int64_t)(s >> 1) * CB, s & 1, lane);
  };
  // Two stages, the next step's loads issued one step ahead: two workgroups
  // share a CU (64 KB of LDS and at most 256 registers per wave each), so
  // one's loads, epilogue and prologue run under the other's multiplies.
  // Blocks are multiplied one at a time (one block's A and B fragments live).
  auto step = [&](auto P_, int s) {  // s: step of this workgroup
    constexpr int P = decltype(P_)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();  // the other stage is free (every wave is past step s - 1)
    if (s + 1 < nsteps) issue(ic<(P + 1) % 2>{}, s + 1);
    if (act) {
      const unsigned char* st = S.get<P>();
      // the A fragment of the next row group is read before the current
      // one's multiplies, so LDS latency hides under them; with 2-bit blocks
      // and at least four row groups the next block's weight fragments are
      // also dequantized between this block's multiplies (one fragment per
      // NRG / 4 row groups) instead of in a burst before them (3-bit and
      // codebook blocks have no registers to spare for the second set)
      constexpr bool SPREAD = BITS == 2 && NRG >= 4;
      half8_t A = *reinterpret_cast<const half8_t*>(st + xs[0]);
      half8_t B[4];
      if constexpr (SPREAD) {
#pragma unroll
        for (int m = 0; m < 4; ++m) B[m] = dequant<BITS>(bw[P][m], 0);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        half8_t Bn[4];
        if constexpr (!SPREAD) {
#pragma unroll
          for (int m = 0; m < 4; ++m) B[m] = dequant<BITS>(bw[P][m], kb);
        }
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
          const bool last = kb == 3 && rg == NRG - 1;
          const int nkb = rg == NRG - 1 ? kb + 1 : kb, nrg = rg == NRG - 1 ? 0 : rg + 1;
          const half8_t An = last ? A : *reinterpret_cast<const half8_t*>(st + nrg * 4096 + xs[nkb & 3]);
          __builtin_amdgcn_sched_barrier(0);  // (the read stays ahead of the multiplies)
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[rg][m] = mfma16x16x32(A, B[m], acc[rg][m]);
          if constexpr (SPREAD) {
            if (kb < 3 && (rg * 4) % NRG == 0) Bn[rg * 4 / NRG] = dequant<BITS>(bw[P][rg * 4 / NRG], kb + 1);
          }
          A = An;
        }
        if constexpr (SPREAD) {
          if (kb < 3) {
#pragma unroll
            for (int m = 0; m < 4; ++m) B[m] = Bn[m];
          }
        }
      }
    }
  };
  issue(ic<0>{}, 0);
  for (int s = 0; s < nsteps; s += 2) {
    step(ic<0>{}, s);
    if (s + 1 < nsteps) step(ic<1>{}, s + 1);
  }

  // epilogue: g, u scaled back by 2^ex of the row's token, h = silu(g) u,
  // stored as fp16(h * 2^-eh) with eh = hb + 2 ex fixed per (expert, row):
  // hb bounds |g| |u| for any input row scaled below 2^15, so h * 2^-eh
  // stays below 2^14 without a pass over the row
  const int hb = a.hb[g];
  __syncthreads();  // every wave is past its last read of stage 0
  uint32_t* tile = reinterpret_cast<uint32_t*>(S.s0);  // fragments [row group][4 blocks]
  if (act)
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rg + 4 * q + i;
        const int ex = ex_lds[r];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // h 2^-eh = silu(g) (u 2^-(hb + ex)): the power of two is applied to
          // u before the product (exact either way), one scaling fewer
          const float gg = ldexpf(acc[rg][j][i], ex);
          const float us = ldexpf(acc[rg][2 + j][i], -(hb + ex));
          const float hv = gg * __builtin_amdgcn_rcpf(1.0f + __expf(-gg)) * us;
          // columns c = 16 j + n and c + 1 (lanes n, n + 1) share one dword:
          // the neighbour's value by a lane swap, both rounded by one packed
          // conversion
          const float hn = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hv), 0xB1, 0xF, 0xF, true));
          if ((n & 1) == 0) {
            const int c = 16 * j + n;
            tile[((rg * 4 + wv) * 64 + 4 * q + i + 16 * (c >> 3)) * 4 + ((c & 7) >> 1)] =
                __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{hv, hn}, half2_t));
          }
        }
      }
  __syncthreads();
  if (act)
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
      if (16 * rg < rows) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(S.s0 + ((rg * 4 + wv) * 64 + lane) * 16);
        *reinterpret_cast<u32x4_t*>(a.hfrag + (((size_t)((row0 >> 4) + rg) * a.nbH + nt * 4 + wv) * 64 + lane) * 8) = v;
      }
}

template <int BITS>
__global__ __launch_bounds__(256, 2) void pf_gate_up_kernel(PfGemmArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char st0[GEMM_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[GEMM_STAGE];
  unsigned char* const st2 = st0;  // (two stages; a third is never used)
  __shared__ int ex_lds[PF_TM];
  load_grid<BITS>(a.X.grid16, threadIdx.x, 256);  // (the first step's barrier publishes it)
  int item, nt;
  // a workgroup without a work item reads the next layer's lines ahead
  // (its share of them: rank blockIdx.x of the grid)
  if (!xcd_tile(*a.n_items, a.n_nt, &item, &nt)) {
    warm_lines(a.warm, blockIdx.x, gridDim.x, st0);
    return;
  }
  const int g = a.item_group[item], row0 = a.item_row0[item], rows = a.item_rows[item];
  const int Ig = g == a.E ? a.Is : a.I;
  if (nt * PF_HT >= Ig) {
    warm_lines(a.warm, blockIdx.x, gridDim.x, st0);
    return;
  }
  const int nrg = rows >> 4;
  const Stages S{st0, st1, st2};
  if (nrg > 4) gate_up_item<BITS, 8>(a, S, ex_lds, g, row0, rows, nt);
  else if (nrg > 2) gate_up_item<BITS, 4>(a, S, ex_lds, g, row0, rows, nt);
  else if (nrg > 1) gate_up_item<BITS, 2>(a, S, ex_lds, g, row0, rows, nt);
  else gate_up_item<BITS, 1>(a, S, ex_lds, g, row0, rows, nt);
}

// ---------------------------------------------------------------------------
// down grouped GEMM.  Workgroup: one work item x 256 output columns; wave wv:
// all rows x output columns r0 = 256 nt + 64 wv .. +64 (4 tiles of 16 rows of
// W_d).  The packed down matrix has row groups of 16 RT rows and k-groups of
// BK blocks (RT BK = 8); per step of 4 blocks the wave holds NC chunk
// registers:
//   BK 8: 4 half chunks (one per row tile),   fragment (t, j) = (c t, f j)
//   BK 4: 2 full chunks (row tiles 2c, 2c+1), fragment (t, j) = (c t/2, f 4(t%2)+j)
//   BK 2: 2 full chunks (blocks 2c, 2c+1),    fragment (t, j) = (c j/2, f 2t+j%2)
//   BK 1: 4 half chunks (one per block),      fragment (t, j) = (c j, f t)
// The intermediate rows are stored in MFMA A-fragment order, so each
// direct-to-LDS load moves 1 KB of consecutive bytes.
// ---------------------------------------------------------------------------
template <int BK>
struct DownMap {
  static constexpr int NC = (BK == 4 || BK == 2) ? 2 : 4;
  static DEVI constexpr int chunk(int t, int j) { return BK == 8 ? t : BK == 4 ? t / 2 : BK == 2 ? j / 2 : j; }
  static DEVI constexpr int frag(int t, int j) { return BK == 8 ? j : BK == 4 ? 4 * (t % 2) + j : BK == 2 ? 2 * t + j % 2 : t; }
};

template <int BITS, int BK, int NRG>
DEVI void down_item(const PfGemmArgs& a, const Stages& S, float* rowf_lds, int g, int row0, int rows, int nt) {
  using M = DownMap<BK>;
  constexpr int RT = 8 / BK;
  static_assert(RT * BK == 8, "chunk shape");
  constexpr int CB = moe_chunk_bytes(BITS);
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 15, q = lane >> 4;
  const bool shared = g == a.E;
  const int Ig = shared ? a.Is : a.I;
  const int nbK = Ig / 32, n_kg = nbK / BK, nsteps = (nbK + 3) / 4;
  const uint8_t* dm =
      (shared ? a.X.shared : a.X.experts + (int64_t)g * a.X.ex_stride) + (shared ? a.X.sh_off_down : a.X.off_down);
  const int r0 = nt * PF_DT + 64 * wv;
  const int nrg = rows >> 4;
  if (tid < rows) {
    const int tok = a.row_tok[row0 + tid];
    const float f = ldexpf(a.row_w[row0 + tid], a.hb[g] + 2 * a.ex[tok] + a.ed[g]);
    rowf_lds[tid] = f;
    if (nt == 0) a.rowf[row0 + tid] = f;
  }
  const int ed = a.ed[g];

  float4_t acc[NRG][4];
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[rg][t] = float4_t{0.f, 0.f, 0.f, 0.f};

  WRegs bw[2][M::NC];
  auto issue = [&](auto P_, int s) {
    constexpr int P = decltype(P_)::value;
    unsigned char* st = S.get<P>();
    // wave wv stages block 4 s + wv of every row group (clamped to valid
    // fragments past the item or the matrix; those are never read)
    const int kb = min(4 * s + wv, nbK - 1);
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const int rgc = rg < nrg ? rg : 0;
      __builtin_amdgcn_global_load_lds(a.hfrag + (((size_t)((row0 >> 4) + rgc) * a.nbH + kb) * 64 + lane) * 8,
                                       (lds_ptr_t)(st + (rg * 4 + wv) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < M::NC; ++c) {
      if constexpr (BK == 8) {
        load_half<BITS>(bw[P][c], dm + ((int64_t)(r0 / 16 + c) * n_kg + (s >> 1)) * CB, s & 1, lane);
      } else if constexpr (BK == 4) {
        load_full<BITS>(bw[P][c], dm + ((int64_t)(r0 / 32 + c) * n_kg + s) * CB, lane);
      } else if constexpr (BK == 2) {
        load_full<BITS>(bw[P][c], dm + ((int64_t)(r0 / 64) * n_kg + min(2 * s + c, n_kg - 1)) * CB, lane);
      } else {
        load_half<BITS>(bw[P][c], dm + ((int64_t)(r0 / 128) * n_kg + min(4 * s + c, n_kg - 1)) * CB, (r0 / 64) & 1, lane);
      }
    }
  };
  // Two stages, the next step's loads issued one step ahead: two workgroups
  // share a CU (64 KB of LDS and at most 256 registers per wave each), so
  // one's loads, epilogue and prologue run under the other's multiplies.
  // Blocks are multiplied one at a time (one block's A and B fragments live).
  auto step = [&](auto P_, int s) {  // s: step of this workgroup
    constexpr int P = decltype(P_)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();  // the other stage is free (every wave is past step s - 1)
    if (s + 1 < nsteps) issue(ic<(P + 1) % 2>{}, s + 1);
    const unsigned char* st = S.get<P>();
    const int nj = min(4, nbK - 4 * s);
    // the A fragment of the next row group is read before the current
    // one's multiplies, so LDS latency hides under them; with 2-bit blocks
    // and at least four row groups the next block's weight fragments are
    // dequantized between this block's multiplies (as in gate/up)
    constexpr bool SPREAD = BITS == 2 && NRG >= 4;
    half8_t A = *reinterpret_cast<const half8_t*>(st + 16 * lane);
    half8_t B[4];
    if constexpr (SPREAD) {
#pragma unroll
      for (int t = 0; t < 4; ++t) B[t] = dequant<BITS>(bw[P][M::chunk(t, 0)], M::frag(t, 0));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nj) break;
      half8_t Bn[4];
      if constexpr (!SPREAD) {
#pragma unroll
        for (int t = 0; t < 4; ++t) B[t] = dequant<BITS>(bw[P][M::chunk(t, j)], M::frag(t, j));
      }
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const bool last = j == 3 && rg == NRG - 1;
        const int nj2 = rg == NRG - 1 ? j + 1 : j, nrg = rg == NRG - 1 ? 0 : rg + 1;
        const half8_t An = last ? A : *reinterpret_cast<const half8_t*>(st + (nrg * 4 + (nj2 & 3)) * 1024 + 16 * lane);
        __builtin_amdgcn_sched_barrier(0);  // (the read stays ahead of the multiplies)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[rg][t] = mfma16x16x32(A, B[t], acc[rg][t]);
        if constexpr (SPREAD) {
          if (j < 3 && (rg * 4) % NRG == 0) {
            const int t = rg * 4 / NRG;
            Bn[t] = dequant<BITS>(bw[P][M::chunk(t, j + 1)], M::frag(t, j + 1));
          }
        }
        A = An;
      }
      if constexpr (SPREAD) {
        if (j < 3) {
#pragma unroll
          for (int t = 0; t < 4; ++t) B[t] = Bn[t];
        }
      }
    }
  };
  issue(ic<0>{}, 0);
  for (int s = 0; s < nsteps; s += 2) {
    step(ic<0>{}, s);
    if (s + 1 < nsteps) step(ic<1>{}, s + 1);
  }
  // rows stored as fp16(sum 2^-ed) (below 2^15, see the pack-time bound);
  // the combine multiplies them by rowf = w 2^(hb + 2 ex + ed).  The tile
  // (rows x 256 columns, 512 B per row) is assembled in LDS, rows 0..63 in
  // stage 0 and 64..127 in stage 1, columns n and n + 1 (lanes n, n ^ 1)
  // sharing one dword, then written out in 16-byte pieces.  Dword c of row r
  // sits at c ^ 8 ((r >> 2) & 3): the four lane groups of a store (rows 4
  // apart, 512 B apart, so the same banks unswizzled) then take distinct
  // banks, and 16-byte pieces stay whole.
  (void)rowf_lds;
  __syncthreads();  // every wave is past its last read of the stages
#pragma unroll
  for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rg + 4 * q + i;
      uint32_t* trow = reinterpret_cast<uint32_t*>((r < 64 ? S.s0 : S.s1) + (r & 63) * 512);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float v = ldexpf(acc[rg][t][i], -ed);
        const float vn = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // lane n ^ 1
        if ((n & 1) == 0)
          trow[((64 * wv + 16 * t + n) >> 1) ^ (8 * ((r >> 2) & 3))] =
              __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{v, vn}, half2_t));
      }
    }
  __syncthreads();
  for (int p = tid; p < rows * 32; p += 256) {
    const int r = p >> 5, c16 = p & 31;
    const u32x4_t v =
        *reinterpret_cast<const u32x4_t*>((r < 64 ? S.s0 : S.s1) + (r & 63) * 512 + 16 * (c16 ^ (2 * ((r >> 2) & 3))));
    *reinterpret_cast<u32x4_t*>(a.yh + (size_t)(row0 + r) * a.d + nt * PF_DT + 8 * c16) = v;
  }
}

template <int BITS, int BK>
__global__ __launch_bounds__(256, 2) void pf_down_kernel(PfGemmArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char st0[GEMM_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[GEMM_STAGE];
  unsigned char* const st2 = st0;  // (two stages; a third is never used)
  __shared__ float rowf_lds[PF_TM];
  load_grid<BITS>(a.X.grid16, threadIdx.x, 256);  // (the first step's barrier publishes it)
  int item, nt;
  if (!xcd_tile(*a.n_items, a.d / PF_DT, &item, &nt)) return;
  const int g = a.item_group[item], row0 = a.item_row0[item], rows = a.item_rows[item];
  const int nrg = rows >> 4;
  const Stages S{st0, st1, st2};
  if (nrg > 4) down_item<BITS, BK, 8>(a, S, rowf_lds, g, row0, rows, nt);
  else if (nrg > 2) down_item<BITS, BK, 4>(a, S, rowf_lds, g, row0, rows, nt);
  else if (nrg > 1) down_item<BITS, BK, 2>(a, S, rowf_lds, g, row0, rows, nt);
  else down_item<BITS, BK, 1>(a, S, rowf_lds, g, row0, rows, nt);
}

// ---------------------------------------------------------------------------
// combine: y[t] = sum over the token's used pairs in rank order + shared row.
// ---------------------------------------------------------------------------
// One wavefront per token (four per workgroup): lane l takes the 8 columns
// 8 l + 512 j of chunk j.  The token's row positions and factors are
// wave-uniform (scalar loads); the K + 1 rows of two chunks (16-byte loads)
// are all issued before the first add.  The sum is formed in rank order, the
// shared row last; skipped entries (position -1) are left out.
template <int K>
__global__ __launch_bounds__(256) void pf_combine_kernel(PfCombineArgs a) {
  constexpr int NR = K + 1;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6)), lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int d = a.d;
  int pos[NR];
#pragma unroll
  for (int r = 0; r < K; ++r) pos[r] = a.slot_pos[(size_t)t * K + r];
  pos[K] = a.has_shared ? a.offsets[a.E] + t : -1;
  float f[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) f[r] = a.rowf[max(pos[r], 0)];
  for (int c0 = 8 * lane; c0 < d; c0 += 1024) {
    const int c1 = min(c0 + 512, d - 8);  // (a second chunk past d re-reads the last columns, not stored)
    half8_t v[2][NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const _Float16* row = a.yh + (size_t)max(pos[r], 0) * d;
      v[0][r] = *reinterpret_cast<const half8_t*>(row + c0);
      v[1][r] = *reinterpret_cast<const half8_t*>(row + c1);
    }
    __builtin_amdgcn_sched_barrier(0);  // (every load issued before the first add)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && c0 + 512 >= d) break;
      float4_t acc0 = float4_t{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (pos[r] >= 0) {
          const half8_t& x = v[h][r];
          acc0 += f[r] * float4_t{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
          acc1 += f[r] * float4_t{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
        }
      float* yo = a.y + (size_t)t * d + (h ? c1 : c0);
      *reinterpret_cast<float4_t*>(yo) = acc0;
      *reinterpret_cast<float4_t*>(yo + 4) = acc1;
    }
  }
}

// ---------------------------------------------------------------------------
// Test export of one packed matrix through the grouped GEMMs' own register
// dequantization: one wavefront per chunk, loaded as two half chunks
// (load_half, as the gate/up kernel and the down kernel with 8 or 1 blocks
// per chunk do) or as one full chunk (load_full, as the down kernel with 4
// or 2 blocks per chunk does), each fragment through dequant.  Lane
// l = n + 16 q writes the fp16 bits of row 16 (RT rg + t) + n, inputs
// 32 (BK kg + j) + 8 q + c of fragment f = BK t + j.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void debug_prefill_path_kernel(DebugPathArgs a) {
  const int chunk = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if constexpr (BITS == MOE_KIND_CB) {
    load_grid<BITS>(a.grid16, threadIdx.x, blockDim.x);
    __syncthreads();
  }
  if (chunk >= a.n_rg * a.n_kg) return;
  const int rg = chunk / a.n_kg, kg = chunk - rg * a.n_kg;
  const int n = lane & 15, q = lane >> 4;
  const uint8_t* ch = a.mat + (int64_t)chunk * a.chunk_bytes;
  auto put = [&](int f, const half8_t& w) {
    const int t = f / a.BK, j = f - t * a.BK;
    const size_t o = (size_t)((rg * a.RT + t) * 16 + n) * a.cols + 32 * (kg * a.BK + j) + 8 * q;
    *reinterpret_cast<half8_t*>(a.w16 + o) = w;  // (o is a multiple of 8: 16-byte aligned)
  };
  if (a.full) {
    WRegs w;
    load_full<BITS>(w, ch, lane);
#pragma unroll
    for (int f = 0; f < 8; ++f) put(f, dequant<BITS>(w, f));
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      WRegs w;
      load_half<BITS>(w, ch, h, lane);
#pragma unroll
      for (int f = 0; f < 4; ++f) put(4 * h + f, dequant<BITS>(w, f));
    }
  }
}

}  // namespace

hipError_t launch_debug_prefill_path(const DebugPathArgs& a, int bits, hipStream_t s) {
  const int n = a.n_rg * a.n_kg;
  if (n == 0) return hipSuccess;
  if (bits == 2) hipLaunchKernelGGL(debug_prefill_path_kernel<2>, dim3((n + 3) / 4), dim3(256), 0, s, a);
  else if (bits == 3) hipLaunchKernelGGL(debug_prefill_path_kernel<3>, dim3((n + 3) / 4), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(debug_prefill_path_kernel<MOE_KIND_CB>, dim3((n + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_router(const float* W, int E, int d, _Float16* wh, _Float16* wl, int32_t* ew, hipStream_t s) {
  const int E16 = (E + 15) / 16 * 16;
  hipLaunchKernelGGL(pack_router_kernel, dim3((E16 + 3) / 4), dim3(256), 0, s, W, E, E16, d, wh, wl, ew);
  return hipGetLastError();
}

hipError_t launch_pack_hbound(const uint8_t* canon, int64_t canon_stride, int n_experts, int I, int d, int bits,
                              const uint8_t* grid, int32_t* hb, int32_t* ed, hipStream_t s) {
  if (n_experts <= 0) return hipSuccess;
  if (bits == MOE_KIND_CB && !grid) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_hbound_kernel, dim3(n_experts), dim3(256), 0, s, canon, canon_stride, I, d, bits, grid, hb,
                     ed);
  return hipGetLastError();
}

hipError_t launch_pf_prep(const PfPrepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(pf_prep_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_router(const PfRouterArgs& a, hipStream_t s, bool reduce) {
  MOE_LAUNCH(pf_router_kernel, dim3((a.T + 127) / 128, (a.E16 + PF_ET - 1) / PF_ET, a.split ? a.d / 256 : 1), dim3(512),
             0, s, a);
  if (a.split && reduce) {
    const int64_t n = (int64_t)a.T * a.E;
    hipLaunchKernelGGL(pf_router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_pf_group(const PfGroupArgs& a, hipStream_t s) {
  if (a.T <= PF_SMALL_T && a.E <= PF_SMALL_E && a.k <= MOE_MAX_K) {
    hipLaunchKernelGGL(pf_group_small_kernel, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(pf_hist_kernel, dim3(a.n_tiles), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pf_scan_kernel, dim3(1), dim3(1024), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = (int64_t)a.T * a.k;
  hipLaunchKernelGGL(pf_permute_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_gate_up(const PfGemmArgs& a, int bits, int max_items, hipStream_t s) {
  const dim3 grid((unsigned)((max_items + N_XCD - 1) / N_XCD * N_XCD * a.n_nt));
  if (bits == 2) MOE_LAUNCH(pf_gate_up_kernel<2>, grid, dim3(256), 0, s, a);
  else if (bits == 3) MOE_LAUNCH(pf_gate_up_kernel<3>, grid, dim3(256), 0, s, a);
  else MOE_LAUNCH(pf_gate_up_kernel<MOE_KIND_CB>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_down(const PfGemmArgs& a, int bits, int bk, int max_items, hipStream_t s) {
  const dim3 grid((unsigned)((max_items + N_XCD - 1) / N_XCD * N_XCD * (a.d / PF_DT)));
#define PF_DOWN(B, K) MOE_LAUNCH((pf_down_kernel<B, K>), grid, dim3(256), 0, s, a)
#define PF_DOWN_BK(B)         \
  switch (bk) {               \
    case 8: PF_DOWN(B, 8); break; \
    case 4: PF_DOWN(B, 4); break; \
    case 2: PF_DOWN(B, 2); break; \
    default: PF_DOWN(B, 1); break; \
  }
  if (bits == 2) {
    PF_DOWN_BK(2)
  } else if (bits == 3) {
    PF_DOWN_BK(3)
  } else {
    PF_DOWN_BK(MOE_KIND_CB)
  }
#undef PF_DOWN_BK
#undef PF_DOWN
  return hipGetLastError();
}

hipError_t launch_pf_combine(const PfCombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.d % 8 != 0 || a.k < 1 || a.k > MOE_MAX_K) return hipErrorInvalidValue;
  const dim3 grid((a.T + 3) / 4), block(256);
  switch (a.k) {
#define MOE_COMBINE_CASE(K) \
  case K: hipLaunchKernelGGL(pf_combine_kernel<K>, grid, block, 0, s, a); break;
    MOE_COMBINE_CASE(1) MOE_COMBINE_CASE(2) MOE_COMBINE_CASE(3) MOE_COMBINE_CASE(4)
    MOE_COMBINE_CASE(5) MOE_COMBINE_CASE(6) MOE_COMBINE_CASE(7) MOE_COMBINE_CASE(8)
    MOE_COMBINE_CASE(9) MOE_COMBINE_CASE(10) MOE_COMBINE_CASE(11) MOE_COMBINE_CASE(12)
    MOE_COMBINE_CASE(13) MOE_COMBINE_CASE(14) MOE_COMBINE_CASE(15) MOE_COMBINE_CASE(16)
#undef MOE_COMBINE_CASE
  }
  return hipGetLastError();
}
