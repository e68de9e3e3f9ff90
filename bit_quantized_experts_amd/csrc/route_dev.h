// route_dev.h -- device code of the decode router (column-sliced router
// GEMV on the matrix cores, logits finished by the last workgroup of each row
// slice), shared by the per-phase route kernel (route.hip) and the
// persistent stack kernel (persist.hip).
//
// The router keeps about ten of 512 small experts per token [cnyes profile of
// Strata, section "Strata 到底是什麼？"]; it stays resident next to the
// shared expert [same page, section "三層記憶體", part 1].
//
// Decode splits the router GEMV over column slices of the input so that no
// workgroup needs the whole input row: the previous layer's output arrives as
// split partial sums, and each workgroup adds only the 128 columns it
// multiplies.  RMSNorm is a per-token scale, so it is applied after the dot
// products (logit = (y . w) / rms(y) + bias) and, in the expert kernels, to
// the accumulators before the SwiGLU nonlinearity.
#pragma once
#include "kern_common.h"
#include "moe_launch.h"

namespace {

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

// Wavefront wv finishes tokens wv + 4j (below T), in passes of NP: every
// load of a pass is issued before its first add, at clamped addresses.  A
// wavefront has at most two tokens up to T = 8 and four up to 16; up to 32
// column slices one pass takes all of them (one round trip whatever T),
// wider inputs take two per pass (the partials of four tokens would not fit
// in registers).
template <int MAXCS, int NP>
DEVI void finish_pass(const RouteArgs& a, int rs, int j0, int nj, int wv, int lane) {
  const SelectArgs& c = a.sel;
  const int T = a.T, E = a.E, n_cs = c.n_cs;
  const int er = rs * MOE_ROUTE_ROWS + lane, e = min(er, E - 1);
  const bool e_ok = er < E;
  const int ew = a.do_logits ? c.ew[e] : 0;
  const float bias = a.do_logits ? c.br[e] : 0.f;
  const float* ssr = c.ss_part + (size_t)rs * n_cs * T;
  float ss[NP], tmp[NP][MAXCS];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int t = min(wv + 4 * min(j0 + j, nj - 1), T - 1);
    ss[j] = ld_dev(ssr + min(lane, n_cs - 1) * T + t);
    if (a.do_logits) {
#pragma unroll
      for (int q = 0; q < MAXCS; ++q) tmp[j][q] = ld_dev(a.lp + ((size_t)min(q, n_cs - 1) * T + t) * E + e);
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (j0 + j >= nj) break;
    const int tok = wv + 4 * (j0 + j);
    const float r = c.norm ? sqrtf(wave_sum((lane < n_cs) ? ss[j] : 0.f) / (float)c.d + c.eps) : 1.0f;
    if (rs == 0 && lane == 0) st_dev(c.rnorm + tok, r);
    if (!a.do_logits) continue;
    float acc = tmp[j][0];
#pragma unroll
    for (int q = 1; q < MAXCS; ++q)
      if (q < n_cs) acc += tmp[j][q];
    const float x = ldexpf(acc, ew);  // router row factor, exact
    const float l = (c.norm ? x / r : x) + bias;
    if (e_ok) {
      st_dev(c.logits + (size_t)tok * c.logits_stride + er, l);
      if (c.out_logits) c.out_logits[(size_t)tok * E + er] = l;
    }
  }
}

template <int MAXCS>
DEVI void finish_slice(const RouteArgs& a, int rs) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wv >= 4) return;  // (four wavefronts finish a slice; no barrier follows here)
  static_assert(MOE_MAX_TOK_F16ACT <= 16, "at most four tokens per wavefront");
  const int nj = (a.T - wv + 3) / 4;  // this wavefront's tokens (wave-uniform)
  if (nj <= 2) {
    if (nj > 0) finish_pass<MAXCS, 2>(a, rs, 0, nj, wv, lane);
  } else if constexpr (MAXCS <= 32) {
    finish_pass<MAXCS, 4>(a, rs, 0, nj, wv, lane);
  } else {
    finish_pass<MAXCS, 2>(a, rs, 0, nj, wv, lane);
    finish_pass<MAXCS, 2>(a, rs, 2, nj, wv, lane);
  }
}

// reset: put the counter back to zero for the next launch (the persistent
// kernel's counters are per layer and cleared before each pass instead).
// With done, the finishing workgroup adds one to it once its logits and
// divisors are stored.
DEVI void route_finish(const RouteArgs& a, int rs, int* flag, bool reset, uint32_t* done) {
  uint32_t* ctr = a.sel.ctrl + (size_t)rs * a.sel.ctrl_stride;
  if (!count_done(ctr, (uint32_t)a.sel.n_cs, flag)) return;
  if (reset && threadIdx.x == 0) *ctr = 0u;
  if (a.sel.n_cs <= 16) finish_slice<16>(a, rs);
  else if (a.sel.n_cs <= 20) finish_slice<20>(a, rs);  // d = 2560
  else if (a.sel.n_cs <= 32) finish_slice<32>(a, rs);
  else finish_slice<64>(a, rs);
  if (done) {
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) signal_add(done);
  }
}

// ---------------------------------------------------------------------------
// Route: workgroup (column slice cs of 128 inputs, row slice rs of 64
// experts).  Sums the input splits for its columns, writes partial logits of
// its 64 experts over those columns and the slice's sums of squares (every
// row slice its own copy); the rs == 0 workgroups also write the slice's
// blocks of the gate/up kernel's A operand (XFrag: the fragments, their
// accumulator seeds and the slice's token exponents) and the caller's copy
// of the summed input if asked.
// The partial logits run on the matrix cores: fp16 hi/lo A-fragments of 8
// tokens of the slice scaled by 2^-e (e per token and slice, from the
// slice's largest magnitude, so the split neither overflows nor underflows;
// a second row tile for tokens 8..15) times the router rows prepared at pack
// time as 2^ew (wh + wl), fp16 hi and lo B-fragments, so one wavefront's 16
// experts over the 4 blocks take 8 v_mfma_f32_16x16x32_f16 and the hi and lo
// rows of a token are added once at the end, then scaled back by 2^e.  All
// four products of the ~22-bit operands are formed exactly; the rounding is
// fp32 accumulation.  The power of two 2^ew of each router row is applied to
// the summed partials (exact) by the workgroup that finishes the row slice
// (above).
// ---------------------------------------------------------------------------
// A-fragment of block bl of the slice: lane L = m + 16q holds row m (m < 8:
// token m, hi part; m >= 8: token m-8, lo part) at inputs 8q..8q+7, scaled by
// 2^-e of its token.
DEVI half8_t x_fragment(const float (*ys)[MOE_ROUTE_COLS], int bl, int lane, int T, int e) {
  const int m = lane & 15, q = lane >> 4, tok = m & 7, lo = m >> 3;  // (ys, T: from the tile's first token)
  float4_t v0 = float4_t{0.f, 0.f, 0.f, 0.f}, v1 = v0;
  if (tok < T) {
    v0 = *reinterpret_cast<const float4_t*>(&ys[tok][32 * bl + 8 * q]);
    v1 = *reinterpret_cast<const float4_t*>(&ys[tok][32 * bl + 8 * q + 4]);
  }
  half8_t h;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float v = ldexpf(c < 4 ? v0[c] : v1[c - 4], -e);  // exact (2^-e itself may exceed the fp32 range)
    const _Float16 hi = (_Float16)v;
    h[c] = lo ? (_Float16)(v - (float)hi) : hi;
  }
  return h;
}

// The same for 16 token rows: lane L = m + 16q holds token m at inputs
// 8q..8q+7, scaled by 2^-e of the token, as its fp16 hi part (in h) and the
// fp16 rest (in lo).
DEVI void x_fragment16(const float (*ys)[MOE_ROUTE_COLS], int bl, int lane, int T, int e, half8_t& h, half8_t& lo) {
  const int m = lane & 15, q = lane >> 4;
  float4_t v0 = float4_t{0.f, 0.f, 0.f, 0.f}, v1 = v0;
  if (m < T) {
    v0 = *reinterpret_cast<const float4_t*>(&ys[m][32 * bl + 8 * q]);
    v1 = *reinterpret_cast<const float4_t*>(&ys[m][32 * bl + 8 * q + 4]);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float v = ldexpf(c < 4 ? v0[c] : v1[c - 4], -e);
    h[c] = (_Float16)v;
    lo[c] = (_Float16)(v - (float)h[c]);
  }
}

// Row slice 0 only: block bl of this column slice as the gate/up kernel's
// A-fragments (device-coherent 16-byte stores: one tile, or the hi and lo
// tiles of 16 tokens) and its accumulator seeds (-2^(b-1) times each row's
// sum of the block's 32 fp16 values, of both tiles with two; four lanes per
// row added), one wavefront per block.
DEVI void write_xfrag(const RouteArgs& a, int cs, const float (*ys)[MOE_ROUTE_COLS], const int* xe, int bl,
                      int lane) {
  const int T = a.T;
  const int b = cs * (MOE_ROUTE_COLS / 32) + bl;
  const __amdgpu_buffer_rsrc_t fr = coh_rsrc(a.x.frag);
  float s = 0.f;
  if (a.am == MOE_AM_HL8) {
    const half8_t A = x_fragment(ys, bl, lane, T, xe[min(lane & 7, T - 1)]);
    coh_st4(fr, (uint32_t)(((size_t)b * 64 + lane) * 16), __builtin_bit_cast(float4_t, A));
#pragma unroll
    for (int c = 0; c < 8; ++c) s += (float)A[c];
  } else {
    half8_t A, Al;
    x_fragment16(ys, bl, lane, T, xe[min(lane & 15, T - 1)], A, Al);
    const int NT = a.am == MOE_AM_HL16 ? 2 : 1;
    coh_st4(fr, (uint32_t)(((size_t)b * NT * 64 + lane) * 16), __builtin_bit_cast(float4_t, A));
    if (NT == 2) coh_st4(fr, (uint32_t)(((size_t)b * NT * 64 + 64 + lane) * 16), __builtin_bit_cast(float4_t, Al));
#pragma unroll
    for (int c = 0; c < 8; ++c) s += (float)A[c];
    if (NT == 2) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s += (float)Al[c];
    }
  }
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  if (lane < 16) st_dev(a.x.cs + (size_t)b * 16 + lane, -(float)a.code_off * s);
}

// One route role (column slice cs, row slice rs) run by the first 256
// threads of the workgroup (others only join the barriers).  In the
// persistent kernel (PERSIST) the router rows are loaded first and stay in
// flight while the workgroup waits until the input slice is ready
// (*wait_ctr >= wait_target; false if the wait gave up), and the finishing
// workgroup adds one to *done; the per-phase kernel loads its input first
// (the previous kernel's output is ready) and resets the row slice's counter.
// ys: [16][128] floats and xe: 16 ints of LDS; flag: a shared int.
template <bool PERSIST>
DEVI bool route_role(const RouteArgs& a, int cs, int rs, float (*ys)[MOE_ROUTE_COLS], int* xe, int* flag,
                     const uint32_t* wait_ctr, uint32_t wait_target, uint32_t* abort_w, uint32_t* done) {
  const int tid = opaque_tid(), lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool active = tid < 256;
  const int T = a.T, d = a.d, E = a.E;
  const int c0 = cs * MOE_ROUTE_COLS;
  constexpr int NBL = MOE_ROUTE_COLS / 32;  // blocks per column slice

  // the input splits of this slice first (the previous kernel's output), then
  // the router fragments of this wave's 16 experts and their row exponents:
  // the wait for the inputs leaves the router loads in flight
  // (every load is issued, rows past T and splits past S_in re-read a valid
  // address, so the wait counts before the first add are exact)
  const int et = rs * (MOE_ROUTE_ROWS / 16) + wv;  // 16-expert tile
  const bool tile_ok = active && a.do_logits && et * 16 < E;
  constexpr int RQ = MOE_ROUTE_COLS / 4;                   // float4 per token row of the slice
  constexpr int PER = (MOE_MAX_TOK_F16ACT * RQ + 255) / 256;  // float4 per thread
  const __amdgpu_buffer_rsrc_t inr = coh_rsrc(a.in);
  float4_t v[PER][MOE_MAX_IN_SPLITS];
  // (every load is issued, rows past T and splits past S_in re-read a valid
  // address, so the wait counts before the first add are exact)
  auto load_input = [&]() {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = (tid & 255) + 256 * j, t = min(i / RQ, T - 1), c4 = i % RQ;  // (rows past T re-read row T - 1)
      const uint32_t off = (uint32_t)((size_t)t * d + c0 + 4 * c4) * 4;
#pragma unroll
      for (int s = 0; s < MOE_MAX_IN_SPLITS; ++s)
        v[j][s] = coh_ld4(inr, off + (uint32_t)((size_t)min(s, a.S_in - 1) * a.in_stride * 4));
    }
  };
  // the router fragments of this wave's 16 experts (issued by every wave,
  // tile 0 standing in for a wave without a tile, so the wait counts stay
  // exact)
  half8_t BH[NBL], BL[NBL];
  auto load_router = [&]() {
    const size_t base = ((size_t)(tile_ok ? et : 0) * (d / 32) + cs * NBL) * 64 * 8;
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      BH[j] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(a.wh + base + ((size_t)j * 64 + lane) * 8));
      BL[j] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(a.wl + base + ((size_t)j * 64 + lane) * 8));
    }
  };
  if constexpr (PERSIST) {
    load_router();
    if (wait_ctr && !wg_wait(wait_ctr, wait_target, abort_w, flag)) return false;
    load_input();
  } else {
    load_input();
    __builtin_amdgcn_sched_barrier(0);  // keep the input loads ahead of the router loads
    load_router();
  }
  // summed input slice into LDS (splits added in order)
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + 256 * j, t = i / RQ, c4 = i % RQ;
    if (active && t < T) {
      float4_t acc = v[j][0];
#pragma unroll
      for (int s = 1; s < MOE_MAX_IN_SPLITS; ++s)
        if (s < a.S_in) acc += v[j][s];
      *reinterpret_cast<float4_t*>(&ys[t][4 * c4]) = acc;
      if (rs == 0 && a.y_out) *reinterpret_cast<float4_t*>(a.y_out + (size_t)t * d + c0 + 4 * c4) = acc;
    }
  }
  __syncthreads();

  // sums of squares of the slice (each row slice keeps its own copy) and its
  // largest magnitude per token
  for (int t = wv; active && t < T; t += 4) {
    const float4 v = lane < RQ ? *reinterpret_cast<const float4*>(&ys[t][4 * lane]) : float4{0.f, 0.f, 0.f, 0.f};
    const float ss = wave_sum(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
    const float mx = wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    if (lane == 0) {
      st_dev(a.sel.ss_part + ((size_t)rs * a.sel.n_cs + cs) * T + t, ss);
      xe[t] = fp16_exponent_for(mx);
    }
  }
  __syncthreads();
  if (rs == 0) {
    static_assert(MOE_ROUTE_COLS == 128, "one wavefront per block of the slice");
    if (active) write_xfrag(a, cs, ys, xe, wv, lane);
    if (tid < 16) st_dev_i(a.x.sx + (size_t)cs * MOE_XSX_STRIDE + tid, tid < T ? xe[tid] : 0);
  }

  if (tile_ok) {
    // row tiles of 8 tokens: tokens 8 tb .. 8 tb + 7
    for (int tb = 0; 8 * tb < T; ++tb) {
      half8_t A[NBL];
      const int tl = min(8 * tb + (lane & 7), T - 1);  // this lane's token (clamped past T: its rows are zero)
#pragma unroll
      for (int j = 0; j < NBL; ++j) A[j] = x_fragment(ys + 8 * tb, j, lane, T - 8 * tb, xe[tl]);
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
        if (lane < 32 && e < E && t < T) st_dev(a.lp + ((size_t)cs * T + t) * E + e, ldexpf(v, xe[t]));
      }
    }
  }
  route_finish(a, rs, flag, !PERSIST, done);
  return true;
}


}  // namespace
