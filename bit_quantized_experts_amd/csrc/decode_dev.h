// decode_dev.h -- device code of the decode path (up to 16 tokens per
// pass), shared by the per-phase kernels (decode.hip) and the persistent
// stack kernel (persist.hip).
//
// Experts are multiplied straight from their low-bit blocks [strata-mlx wiki,
// opening feature list, first item]; one pass checks up to eight tokens (one
// real token and seven drafts) [devlabs blog "32GB Mac mini 6 跑 125B 大模型",
// section 核心技术特点, MTP item].
//
// Arithmetic on the matrix cores (v_mfma_f32_16x16x32_f16), transposed so the
// tokens are the M dimension and weight rows the N dimension:
//   A[m][k]  = activation fp16, m < 8: hi part of token m, m >= 8: lo part
//              of token m-8 (x = hi + lo to ~22 bits, after an exact
//              power-of-two scaling per token),
//   B[k][n]  = unsigned code q of weight row n, input k (exact fp16 integer),
//   C_in[m]  = -2^(b-1) * sum_k A[m][k]  (the block sum, fp32),
// so one MFMA per 32-weight block gives sum_k A (q - 2^(b-1)) = sum_k A c for
// 16 rows; the lane holding column n then applies the fp16 block scale of row
// n with one fused multiply-add per output.  Every product and the offset are
// exact; the rounding is the fp32 accumulation.
// With 9..16 tokens (MOE_AM_HL16) the rows are the 16 tokens: a first MFMA
// with their fp16 hi parts and a second one, chained on the same
// accumulators, with their lo parts, so every weight fragment serves 16
// tokens at full precision; the seed then holds the sums of hi and lo.  With
// fp16 activations (MOE_AM_F16) only the first of the two runs.
//
// Memory: weight chunks stream from HBM into registers, several k-groups
// ahead of the multiplies; the gate/up activation fragments are read from
// LDS (one copy per workgroup).  Everything one workgroup hands to another
// (the layer input, logits, h, the down partials) is stored
// device-coherently (kern_common.h: written through to memory), so the same
// code serves kernels separated by launches and phases of one persistent
// kernel.  The bulk of it (layer input, logits, divisors, exponents, h) is
// read with ordinary, L2-cached loads: a consumer reads such a buffer only
// after its producers have counted it complete, and the persistent kernel
// gives every layer its own copies, so no XCD's L2 can hold an older line of
// them (a kernel starts with its L2 invalidated); the many workgroups that
// read the same line then share one fetch per XCD instead of each going to
// memory.  Values that are rewritten within a kernel and read by few
// workgroups (split partials, partial logits, counters) are loaded
// device-coherently.
#pragma once
#include "kern_common.h"
#include "moe_launch.h"
#include "topk.h"

namespace {

// A lane's share of one chunk.  b-bit kinds: codes (16 B), the 8 fp16
// scales of its row, and for 3 bits the high bits (8 B).  Codebook: index
// bytes (in codes), scales, sign bits (in hbits) and index high bits (hi).
template <int BITS>
struct ChunkRegs {
  u32x4_t codes;
  u32x4_t scales;  // 8 fp16
  u32x2_t hbits;   // 3-bit: high code bits; codebook: sign bits
  uint32_t hi;     // codebook: index high bits
};

template <int BITS>
DEVI void load_chunk(ChunkRegs<BITS>& c, const uint8_t* chunk, int lane) {
  c.codes = ld128_nt(chunk + 16 * lane);
  c.scales = ld128_nt(chunk + 1024 + 16 * (lane & 15));
  if constexpr (BITS != 2) c.hbits = ld64_nt(chunk + 1280 + 8 * lane);
  if constexpr (BITS == MOE_KIND_CB)
    c.hi = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(chunk + 1792 + 2 * lane));
}

template <int BITS>
DEVI half8_t chunk_frag(const ChunkRegs<BITS>& c, int f) {
  if constexpr (BITS == 2) return frag_q2(c.codes, f);
  else if constexpr (BITS == 3) return frag_q3(c.codes, c.hbits, f);
  else return frag_cb(c.codes, c.hi, c.hbits, f, cb_grid_lds);
}

DEVI float chunk_scale(const u32x4_t& s, int f) {
  const uint32_t dw = s[f >> 1];
  return half_bits_to_float((f & 1) ? (dw >> 16) : (dw & 0xffffu));
}

// ---------------------------------------------------------------------------
// Slot list in LDS: routed experts numbered in ascending id order after the
// shared expert's slot 0, and every (token, rank) entry's gate weight in its
// slot's row.  The weight rows are cleared first (the shared expert's row set
// to 1 for the tokens present).  Each token's wavefront marks its experts in
// a byte map (plain byte stores of 1, so no atomics).  After a barrier every
// token's wavefront reads the whole map, one ballot per 64 ids, which gives
// the slot of any marked id (the shared slot plus the marked ids below it),
// and writes its own entries: the slot's expert id and the token's weight.
// Tokens that share an expert write the same id to its slot.
// ---------------------------------------------------------------------------
struct SlotLds {
  uint8_t sel[MOE_MAX_E];  // 1 = selected
  int expert[MOE_MAX_SLOTS];
  float w[MOE_MAX_SLOTS][16];  // [slot][token]
  int n_routed;
};

// Clears the byte map and the first n_slots weight rows (every thread of the
// workgroup takes part).
DEVI void clear_slots(SlotLds& S, int E, int T, int n_slots, bool has_shared) {
  for (int i = threadIdx.x; i < (E + 3) / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(S.sel)[i] = 0u;
  for (int i = threadIdx.x; i < n_slots * 16; i += blockDim.x) (&S.w[0][0])[i] = (has_shared && i < T) ? 1.0f : 0.f;
}

// Marks this lane's expert e (ids out of range are skipped).
DEVI void mark_lane(SlotLds& S, int e, int E) {
  if (e >= 0 && e < E) S.sel[e] = 1;
}

// Token t's wavefront, after every mark: lane r < k holds the token's entry
// (e, w).  Puts w in row t of e's slot and the id in the slot table.  With
// dedup (given routing rows) a repeated id in the row keeps its first entry
// (a selection has no repeats).  With count, lane 0 also writes the number of
// routed slots and the shared expert's slot entry.
template <int NPER>
DEVI void place_lane(SlotLds& S, int e, float w, int t, int k, int E, int base, bool dedup, bool count) {
  const int lane = opaque_tid() & 63;
  uint8_t f[NPER];  // every read first (a guarded read would wait on its own)
#pragma unroll
  for (int i = 0; i < NPER; ++i) f[i] = S.sel[min(lane + 64 * i, E - 1)];
  uint64_t M[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) M[i] = __ballot((f[i] != 0) & (lane + 64 * i < E));
  const bool valid = lane < k && e >= 0 && e < E;
  bool use = valid;
  if (dedup)
    for (int j = 0; j + 1 < k; ++j) use = use && !(j < lane && __builtin_amdgcn_readlane(e, j) == e);
  const int g = valid ? e >> 6 : 0;
  const uint64_t below = valid ? (1ull << (e & 63)) - 1ull : 0ull;
  int slot = base, total = 0;
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int c = (int)__builtin_popcountll(M[i]);
    slot += i < g ? c : 0;
    m = i == g ? M[i] : m;
    total += c;
  }
  slot += (int)__builtin_popcountll(m & below);
  if (valid) S.expert[slot] = e;
  if (use) S.w[slot][t] = w;
  if (count && lane == 0) {
    S.n_routed = total;
    if (base) S.expert[0] = E;
  }
}

// ---------------------------------------------------------------------------
// gate/up: a work item is (slot u, tile t of 16 intermediate rows); slot 0
// is the shared expert when there is one, and its tiles come first.  One
// workgroup of 8 wavefronts per CU (the grid is the CU count): it copies the
// activation fragments and block sums of the input into LDS once (one copy
// serves all of its items), selects every token's experts (or takes the
// given routing rows) and builds the slot list, and then takes its items in
// rounds.  In a round, each item has KP wavefronts
// that take every KP-th k-group (256 inputs) of it, KP in {1, 2, 4, 8} being
// the largest that still gives every wavefront of the grid work.  A wavefront
// keeps the gate and up chunks of two k-groups in flight ahead of the one it
// multiplies.  The KP partial sums are added in k-part order through LDS; the
// epilogue divides by the token's rms (stacked layers), forms h = silu(g) * u
// times the token's gate weight and writes it as fp16 hi/lo A-fragments of
// the down projection, with the sums of each 16-row tile.
// Inputs wider than GU_WIN blocks (GU_WIN / 2 with the two tiles of 16 hi +
// lo token rows, so d = 2560 takes two) are staged in windows, one after
// another.
// ---------------------------------------------------------------------------
constexpr int GU_NW = 8;    // wavefronts per workgroup
constexpr int GU_WIN = 96;  // activation blocks staged in LDS at once

struct alignas(16) GuLds {
  alignas(16) unsigned char xs[GU_WIN * 1024];  // A-fragments, [block][lane][8] fp16
  alignas(16) float cs[GU_WIN * 16];  // accumulator seeds, [block][16]
  float red[GU_NW][8][64];          // partial sums of the k-parts
  float rn[16];                     // 1 / rms of each token
  int sx[MOE_MAX_CS][16];           // exponent e of each (column slice, token) scaling of the fragments
  SlotLds S;
  uint64_t tk_buf[GU_NW][TOPK_BUF];
  int flag;                         // workgroup-wide result of a wait or a count
  int xe[16];                       // route: exponent of each token in the column slice
};

template <int BITS>
struct GroupRegs {
  ChunkRegs<BITS> g, u;
};

// C rows are the 16 tokens themselves (no hi/lo row pairs to add).
constexpr bool am_tok16(int am) { return am != MOE_AM_HL8; }
// Activation windows of the gate/up kernel: a block takes NT KB of LDS.
constexpr int gu_win_blocks(int am) { return GU_WIN / moe_am_tiles(am); }
template <int AM>
DEVI int gu_windows(int n_kg) {
  return (8 * n_kg + gu_win_blocks(AM) - 1) / gu_win_blocks(AM);
}

// Activation blocks [b0, b0 + nblk) of the layer input into LDS: the
// A-fragments (1 KB per tile, NT tiles per block) and accumulator seeds (16
// floats per block) the router wrote (XFrag), copied as 16-byte pieces
// (thread p takes pieces p, p + 512, ...).  Every load is issued unconditionally (pieces past the
// window re-read a valid address and are not stored), so a thread's loads
// stay in flight together.
struct WindowRegs {
  static constexpr int PER = GU_WIN * 64 / (64 * GU_NW);  // fragment pieces per thread
  u32x4_t v[PER];
  float4_t c;  // a piece of the seeds (threads below 4 nblk)
};

template <int AM>
DEVI void window_load(WindowRegs& W, const GuArgs& a, int b0, int nblk, int tid) {
  constexpr int NT = moe_am_tiles(AM);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.x.frag) + (size_t)b0 * NT * 64;
#pragma unroll
  for (int i = 0; i < WindowRegs::PER; ++i) W.v[i] = src[min(tid + 64 * GU_NW * i, 64 * NT * nblk - 1)];
  W.c = reinterpret_cast<const float4_t*>(a.x.cs + (size_t)b0 * 16)[min(tid, 4 * nblk - 1)];
}

template <int AM>
DEVI void window_store(const WindowRegs& W, GuLds& L, int nblk, int tid) {
  constexpr int NT = moe_am_tiles(AM);
#pragma unroll
  for (int i = 0; i < WindowRegs::PER; ++i) {
    const int p = tid + 64 * GU_NW * i;
    if (p < 64 * NT * nblk) *reinterpret_cast<u32x4_t*>(L.xs + (size_t)p * 16) = W.v[i];
  }
  if (tid < 4 * nblk) *reinterpret_cast<float4_t*>(L.cs + 4 * tid) = W.c;
}

template <int AM>
DEVI void stage_window(GuLds& L, const GuArgs& a, int b0, int nblk, int tid) {
  WindowRegs W;
  window_load<AM>(W, a, b0, nblk, tid);
  window_store<AM>(W, L, nblk, tid);
}

template <int BITS>
DEVI void issue_group(GroupRegs<BITS>& r, const uint8_t* gate, const uint8_t* up, int64_t off, int lane) {
  load_chunk<BITS>(r.g, gate + off, lane);
  load_chunk<BITS>(r.u, up + off, lane);
}

// Eight blocks (k-group kg) of gate and up; lb = its first block in the
// window.  A k-group spans two column slices of the router (4 blocks each):
// each slice's sum is scaled back by 2^e of its (slice, token) (exact) before
// it joins the accumulators; this lane's C rows are tokens tok4 .. tok4 + 3.
// (MOE_AM_HL16: the block's lo tile follows its hi tile in LDS, and its
// MFMAs continue the hi tile's accumulators.)
template <int BITS, int AM>
DEVI void mul_group(const GroupRegs<BITS>& r, const GuLds& L, int lb, int kg, int lane, float4_t& accg,
                    float4_t& accu) {
  static_assert(MOE_ROUTE_COLS == 128, "two column slices per k-group");
  constexpr int NT = moe_am_tiles(AM);
  const int tok4 = am_tok16(AM) ? 4 * (lane >> 4) : 4 * ((lane >> 4) & 1);
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    float4_t pg = float4_t{0.f, 0.f, 0.f, 0.f}, pu = pg;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * hs + jj;
      const unsigned char* ap = L.xs + (size_t)(lb + j) * NT * 1024 + 16 * lane;
      const half8_t A = *reinterpret_cast<const half8_t*>(ap);
      const float4_t cin = *reinterpret_cast<const float4_t*>(L.cs + (lb + j) * 16 + 4 * (lane >> 4));
      const half8_t Bg = chunk_frag<BITS>(r.g, j), Bu = chunk_frag<BITS>(r.u, j);
      float4_t Cg = mfma16x16x32(A, Bg, cin);
      float4_t Cu = mfma16x16x32(A, Bu, cin);
      if constexpr (AM == MOE_AM_HL16) {
        const half8_t Al = *reinterpret_cast<const half8_t*>(ap + 1024);
        Cg = mfma16x16x32(Al, Bg, Cg);
        Cu = mfma16x16x32(Al, Bu, Cu);
      }
      pg += chunk_scale(r.g.scales, j) * Cg;
      pu += chunk_scale(r.u.scales, j) * Cu;
    }
    const int4 e = *reinterpret_cast<const int4*>(&L.sx[2 * kg + hs][tok4]);
    accg[0] += ldexpf(pg[0], e.x);
    accg[1] += ldexpf(pg[1], e.y);
    accg[2] += ldexpf(pg[2], e.z);
    accg[3] += ldexpf(pg[3], e.w);
    accu[0] += ldexpf(pu[0], e.x);
    accu[1] += ldexpf(pu[1], e.y);
    accu[2] += ldexpf(pu[2], e.z);
    accu[3] += ldexpf(pu[3], e.w);
  }
}

// k-groups kg0, kg0 + step, ... below kg1 of one 16-row tile (chunk row
// offset rowoff); the window starts at k-group wkg0.  A three-slot register
// ring: each step of the main loop issues the k-group two steps ahead (the
// last k-group again once past the end) and multiplies the oldest one; the
// main loop has no early exit, so the loads in flight at every multiply are
// the same and the compiler's wait counts stay exact; a tail of up to two
// steps multiplies what is already in flight.
template <int BITS, int AM>
DEVI void run_tile(const uint8_t* gate, const uint8_t* up, int64_t rowoff, int kg0, int kg1, int step, int wkg0,
                   const GuLds& L, int lane, float4_t& accg, float4_t& accu) {
  constexpr int64_t CB = moe_chunk_bytes(BITS);
  if (kg0 >= kg1) return;
  const int nsteps = (kg1 - 1 - kg0) / step + 1;
  const int last = kg0 + (nsteps - 1) * step;
  GroupRegs<BITS> r0, r1, r2;
  int kg = kg0;
  issue_group<BITS>(r0, gate, up, rowoff + kg * CB, lane);
  issue_group<BITS>(r1, gate, up, rowoff + min(kg + step, last) * CB, lane);
  __builtin_amdgcn_sched_barrier(0);
  for (int it = nsteps / 3; it > 0; --it) {
    issue_group<BITS>(r2, gate, up, rowoff + min(kg + 2 * step, last) * CB, lane);
    __builtin_amdgcn_sched_barrier(0);
    mul_group<BITS, AM>(r0, L, 8 * (kg - wkg0), kg, lane, accg, accu);
    kg += step;
    issue_group<BITS>(r0, gate, up, rowoff + min(kg + 2 * step, last) * CB, lane);
    __builtin_amdgcn_sched_barrier(0);
    mul_group<BITS, AM>(r1, L, 8 * (kg - wkg0), kg, lane, accg, accu);
    kg += step;
    issue_group<BITS>(r1, gate, up, rowoff + min(kg + 2 * step, last) * CB, lane);
    __builtin_amdgcn_sched_barrier(0);
    mul_group<BITS, AM>(r2, L, 8 * (kg - wkg0), kg, lane, accg, accu);
    kg += step;
  }
  const int rem = nsteps % 3;
  if (rem >= 1) mul_group<BITS, AM>(r0, L, 8 * (kg - wkg0), kg, lane, accg, accu);
  if (rem == 2) mul_group<BITS, AM>(r1, L, 8 * (kg + step - wkg0), kg + step, lane, accg, accu);
}

// Selection and slot list of a gate/up workgroup (every workgroup runs it):
// each token's top k (or the given routing rows), the slot list in LDS, the
// first activation window staged.  publish_routing: write the routing used to the
// caller's outputs; publish_slots: write the slot list to the workspace (for
// a separate down kernel).
template <int BITS, int NPER, int AM>  // NPER >= ceil(E / 64)
DEVI void gu_select(const GuArgs& a, GuLds& L, bool publish_routing, bool publish_slots) {
  const int tid = opaque_tid(), lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: loop bounds stay scalar
  const int T = a.T, k = a.k, E = a.E, tk = a.T * a.k;
  const bool has_shared = a.has_shared != 0;
  const int base = has_shared ? 1 : 0;
  const int n_kg = a.n_kg;
  const int n_win = gu_windows<AM>(n_kg);

  // Selection: wavefront w takes the rows of tokens w and w + 8 (below T) of
  // the logits.  The loads of its first row (both rows, for rows of up to
  // 1024 experts), the divisors' and the activation window's share one round
  // trip.
  constexpr bool PRE2 = NPER <= 16;
  const bool select = a.logits != nullptr;
  float lv[2][NPER];
  if (select) {
#pragma unroll
    for (int h = 0; h < (PRE2 ? 2 : 1); ++h) {
      const float* row = a.logits + (size_t)min(wv + GU_NW * h, T - 1) * a.logits_stride;
#pragma unroll
      for (int i = 0; i < NPER; ++i) lv[h][i] = row[min(lane + 64 * i, E - 1)];
    }
  }
  const float rnv = (tid >= 64 && tid < 64 + T) ? a.rnorm[tid - 64] : 1.0f;
  // the fragments' exponents of every (column slice, token)
  const int n_sx = 16 * (a.d / MOE_ROUTE_COLS);
  int sxv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = min(tid + 512 * h, n_sx - 1);
    sxv[h] = a.x.sx[(size_t)(i >> 4) * MOE_XSX_STRIDE + (i & 15)];
  }
  // the first activation window (the whole input for inputs of up to
  // gu_win_blocks(AM) blocks) stays in registers through the selection and
  // is stored to LDS before the barrier that ends it: the selection starts as
  // soon as its logits are in, while the larger window is still arriving
  const int win_kg = (n_kg + n_win - 1) / n_win;
  WindowRegs win;
  window_load<AM>(win, a, 0, 8 * win_kg, tid);
  clear_slots(L.S, E, T, base + min(tk, E), has_shared);
  lds_barrier();  // byte map and weight rows cleared before any wavefront marks (the loads stay in flight)
  static_assert(2 * GU_NW >= MOE_MAX_TOK_F16ACT, "two tokens per wavefront");
  TopkLane mine[2] = {{-1, 0.f}, {-1, 0.f}};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wv + GU_NW * h;
    if (t < T) {
      if (select) {
        if (!PRE2 && h == 1) {
          const float* row = a.logits + (size_t)t * a.logits_stride;
#pragma unroll
          for (int i = 0; i < NPER; ++i) lv[1][i] = row[min(lane + 64 * i, E - 1)];
        }
        uint64_t key[NPER];
#pragma unroll
        for (int i = 0; i < NPER; ++i) key[i] = (lane + 64 * i < E) ? sel_key(lv[h][i], lane + 64 * i) : 0ull;
        mine[h] = topk_keys<NPER>(key, E, k, nullptr, nullptr, L.tk_buf[wv]);
      } else if (lane < k) {
        mine[h].e = a.idx[t * k + lane];
        mine[h].w = a.w[t * k + lane];
      }
      mark_lane(L.S, mine[h].e, E);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // (the window's stores stay after the selection)
  window_store<AM>(win, L, 8 * win_kg, tid);
  if (tid >= 64 && tid < 80) L.rn[tid - 64] = 1.0f / rnv;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (tid + 512 * h < n_sx) (&L.sx[0][0])[tid + 512 * h] = sxv[h];
  lds_barrier();  // every token's experts marked, the window staged
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wv + GU_NW * h;
    if (t < T) {
      place_lane<NPER>(L.S, mine[h].e, mine[h].w, t, k, E, base, !select, t == 0);
      if (publish_routing && lane < k) {  // the routing used (given rows are copied as they are)
        if (a.out_idx) a.out_idx[t * k + lane] = mine[h].e;
        if (a.out_w) a.out_w[t * k + lane] = mine[h].w;
      }
    }
  }
  lds_barrier();  // slot list, rms and the staged activations
  if (publish_slots) {
    const int ns = base + L.S.n_routed;
    if (tid == 0) *a.n_slots = ns;
    for (int i = tid; i < ns; i += blockDim.x) a.slot_expert[i] = L.S.expert[i];
    for (int i = tid; i < ns * 16; i += blockDim.x) a.slot_w[i] = L.S.w[i >> 4][i & 15];
  }
}

// Workgroups that run only the shared expert's items need no selection:
// their prologue loads the divisors, the slice exponents and the first
// activation window, as gu_select does for the others.
template <int AM>
DEVI void gu_prologue_shared(const GuArgs& a, GuLds& L) {
  const int tid = opaque_tid();
  const int T = a.T, n_kg = a.n_kg, n_win = gu_windows<AM>(n_kg);
  const float rnv = (tid >= 64 && tid < 64 + T) ? a.rnorm[tid - 64] : 1.0f;
  const int n_sx = 16 * (a.d / MOE_ROUTE_COLS);
  int sxv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = min(tid + 512 * h, n_sx - 1);
    sxv[h] = a.x.sx[(size_t)(i >> 4) * MOE_XSX_STRIDE + (i & 15)];
  }
  const int win_kg = (n_kg + n_win - 1) / n_win;
  WindowRegs win;
  window_load<AM>(win, a, 0, 8 * win_kg, tid);
  window_store<AM>(win, L, 8 * win_kg, tid);
  if (tid >= 64 && tid < 80) L.rn[tid - 64] = 1.0f / rnv;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (tid + 512 * h < n_sx) (&L.sx[0][0])[tid + 512 * h] = sxv[h];
  lds_barrier();  // the window, divisors and exponents are staged
}

// The gate/up work items of one workgroup (wg of n_wg): a work item is
// (slot u, tile t of 16 intermediate rows).  With h_ready, each finished
// item adds one to its slot's counter (h_ready + u * MOE_CTR_STRIDE) once its
// h values are stored (a consumer inside the same kernel waits on them).
template <int BITS, int AM>
DEVI void gu_items(const GuArgs& a, GuLds& L, int wg, int n_wg, uint32_t* h_ready, int cls = 0) {
  constexpr int64_t CB = moe_chunk_bytes(BITS);
  const int tid = opaque_tid(), lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T;
  const bool has_shared = a.has_shared != 0;
  const int base = has_shared ? 1 : 0;
  const int tiles_r = a.I / 16, tiles_s = has_shared ? a.Is / 16 : 0;
  const int n_kg = a.n_kg;
  const int n_win = gu_windows<AM>(n_kg);
  const int win_kg = (n_kg + n_win - 1) / n_win;  // k-groups per window
  // items of this call: cls 0 all (shared first), 1 the shared expert's only
  // (no slot list needed), 2 the routed experts' only
  const int i_lo = cls == 2 ? tiles_s : 0;
  const int i_hi = cls == 1 ? tiles_s : tiles_s + L.S.n_routed * tiles_r;
  const int n_items = i_hi - i_lo;
  int KP = 8;
  while (KP > 1 && (KP > n_kg || n_items * KP > n_wg * GU_NW)) KP >>= 1;
  const int G = GU_NW / KP, jw = wv / KP, kp = wv - jw * KP;
  const int tok_e = 4 * ((lane >> 4) & 1);
  int staged = 0;  // the window in LDS (gu_select stages the first)

  for (int grp = wg; grp * G < n_items; grp += n_wg) {
    const int item = i_lo + grp * G + jw;
    const bool valid = item < i_hi;
    int u = 0, t = 0;
    const uint8_t* gate = nullptr;
    const uint8_t* up = nullptr;
    if (valid) {
      const uint8_t* ebase;
      int64_t og, ou;
      if (item < tiles_s) {
        t = item;
        ebase = a.X.shared;
        og = a.X.sh_off_gate;
        ou = a.X.sh_off_up;
      } else {
        const int ri = item - tiles_s;
        u = base + ri / tiles_r;
        t = ri - (ri / tiles_r) * tiles_r;
        ebase = a.X.experts + (int64_t)L.S.expert[u] * a.X.ex_stride;
        og = a.X.off_gate;
        ou = a.X.off_up;
      }
      gate = ebase + og;
      up = ebase + ou;
    }
    float4_t accg = float4_t{0.f, 0.f, 0.f, 0.f}, accu = accg;
    // (several windows: every other round takes them in reverse order, so
    // a round starts with the window the previous round ended with, which
    // is still staged)
    const bool rev = (((grp - wg) / n_wg) & 1) != 0;
    for (int wi = 0; wi < n_win; ++wi) {
      const int w = rev ? n_win - 1 - wi : wi;
      const int kg0 = w * win_kg, kg1 = min(n_kg, kg0 + win_kg);
      if (w != staged) {
        __syncthreads();
        stage_window<AM>(L, a, 8 * kg0, 8 * (kg1 - kg0), tid);
        __syncthreads();
        staged = w;
      }
      // k-group g goes to k-part g % KP in every window, so the parts stay
      // within one k-group of each other however the windows split
      const int first = kg0 + (kp - kg0 % KP + KP) % KP;
      if (valid) run_tile<BITS, AM>(gate, up, (int64_t)t * n_kg * CB, first, kg1, KP, kg0, L, lane, accg, accu);
    }
    if (KP > 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L.red[wv][i][lane] = accg[i];
        L.red[wv][4 + i][lane] = accu[i];
      }
      __syncthreads();
    }
    if (valid) {
      // lane l: intermediate row n = l & 15 of the tile, C rows 4(l>>4)+i:
      // tokens tok_e + i, hi part in lanes < 32, lo part in lanes >= 32 (16
      // token rows: token 4(l>>4)+i, hi and lo already summed).  h is kept in fp32 as
      // [slot][16-row tile][token][16] (an item writes whole 128-byte lines,
      // none shared with another item, zeros for tokens without this slot);
      // the down kernel scales it before rounding to fp16.
      const int n = lane & 15;
      constexpr bool T16 = am_tok16(AM);
      const bool writer = T16 || lane < 32;
      constexpr int R = moe_am_tokens(AM);
      float* hrow = a.hbuf + ((size_t)u * (a.hI / 16) + t) * R * 16 + n;
      // The item's KP waves share the epilogue: wave kp finishes the
      // accumulator rows i with i % KP == kp, summing the k-parts in wave
      // order (KP is a power of two, so the choice is wave-uniform).
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((i & (KP - 1)) != kp) continue;
        float sg = accg[i], su = accu[i];
        if (KP > 1) {
          const int w0 = jw * KP;
          sg = L.red[w0][i][lane];
          su = L.red[w0][4 + i][lane];
          for (int p = 1; p < KP; ++p) {
            sg += L.red[w0 + p][i][lane];
            su += L.red[w0 + p][4 + i][lane];
          }
        }
        const int tok = T16 ? 4 * (lane >> 4) + i : tok_e + i;
        const float gw = (u == 0 && has_shared) ? (tok < T ? 1.0f : 0.f) : L.S.w[u][tok];
        // the norm's 1 / rms (the fragments' scaling was undone per slice)
        const float rrn = L.rn[tok];
        const float g = (T16 ? sg : add_partner32(sg)) * rrn;
        const float uu = (T16 ? su : add_partner32(su)) * rrn;
        const float hv = g * __builtin_amdgcn_rcpf(1.0f + expf(-g)) * uu;
        const float hs = (gw != 0.f) ? gw * hv : 0.f;
        if (writer) st_dev(hrow + tok * 16, hs);
      }
      if (h_ready) __builtin_amdgcn_s_waitcnt(0);  // this wave's h values are stored
    }
    if (KP > 1) __syncthreads();  // red is rewritten in the next round; every wave's stores waited for
    if (h_ready && valid && kp == 0 && lane == 0) signal_add(h_ready + (size_t)u * MOE_CTR_STRIDE);
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
// A-fragment of one block of slot u's intermediate h (fp32 rows
// [slot][token][row]): lane L = m + 16q holds inputs 8q..8q+7 of row m, i.e.
// token m & 7, its fp16 hi part for m < 8 and lo part for m >= 8 (16 token
// rows: token m, its fp16 hi part in h and, for MOE_AM_HL16, its lo part in
// hl), after scaling by the power of two 2^-eh that puts the token's largest
// |h| over the down item's inputs in [2^14, 2^15).
template <int AM>
DEVI void h_fragment(const float4_t (&v)[2], int eh, int lane, half8_t& h, half8_t& hl) {
  const bool lo = AM == MOE_AM_HL8 && (lane & 8);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float x = ldexpf(v[c >> 2][c & 3], -eh);  // exact (2^-eh itself may exceed the fp32 range)
    const _Float16 hi = (_Float16)x;
    const _Float16 rest = (_Float16)(x - (float)hi);
    h[c] = lo ? rest : hi;
    hl[c] = rest;
  }
}

// One down role (row group rg, split sp): ns slots, their expert ids in
// `slots` (the workspace or the workgroup's own LDS slot list); `red` is
// 8 x RT*4 x 64 floats of LDS.  Ends with a barrier (red is free again).
template <int BITS, int RT, int AM>
DEVI void down_role(const DownArgs& a, int rg, int sp, int ns, const int* slots, float* red) {
  constexpr int CB = moe_chunk_bytes(BITS);
  constexpr int BK = 8 / RT;
  constexpr int BATCH = 2;
  constexpr int R = moe_am_tokens(AM);
  constexpr bool T16 = am_tok16(AM);
  const int tid = opaque_tid();
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;
  const int S = a.S;
  // slots of this split: sp, sp + S, ...; slot 0 is the shared expert when
  // there is one (split 0 then starts with its k-groups)
  const bool sh_here = a.has_shared && sp == 0;
  const int first_r = sh_here ? S : sp;  // first routed slot of the split
  const int n_sh = sh_here ? a.n_kg_s : 0;
  // expert ids of this wave's first batch, fetched together with n_slots
  // (the slot of an item does not depend on n_slots; ids past the list are
  // clamped to a valid expert and never used)
  // (two named registers: an array here was kept in scratch memory, and its
  // store waited for the loads)
  static_assert(BATCH == 2, "two prefetched ids");
  int pre0, pre1;
  {
    const int it0 = wv, it1 = wv + nw;
    const int u0 = (it0 < n_sh) ? 0 : first_r + S * ((it0 - n_sh) / a.n_kg_r);
    const int u1 = (it1 < n_sh) ? 0 : first_r + S * ((it1 - n_sh) / a.n_kg_r);
    pre0 = slots[min(u0, a.max_slots - 1)];
    pre1 = slots[min(u1, a.max_slots - 1)];
  }
  const int n_rs = (first_r < ns) ? (ns - first_r + S - 1) / S : 0;
  const int n_items = n_sh + n_rs * a.n_kg_r;

  float4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // this lane's A-fragment token, and the token of its accumulator rows
  // 4 (lane >> 4) + i (hi/lo: the lo rows 8..15 are tokens 0..7 again)
  const int tok_a = T16 ? (lane & 15) : (lane & 7);
  const int tok_c = T16 ? 4 * (lane >> 4) : (4 * (lane >> 4)) & 7;
  const float off = -(float)moe_code_offset(BITS);
  const half8_t ones = half8_t{1, 1, 1, 1, 1, 1, 1, 1};

  for (int b0 = wv; b0 < n_items; b0 += nw * BATCH) {
    ChunkRegs<BITS> c[BATCH];
    float4_t hv[BATCH][BK][2];
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
        int e = (b0 == wv) ? ((ok[q] && q == 1) ? pre1 : pre0) : slots[u];
        e = min(max(e, 0), a.E - 1);
        mat = a.X.experts + (int64_t)e * a.X.ex_stride + a.X.off_down;
      }
      load_chunk<BITS>(c[q], mat + ((int64_t)rg * n_kg + kg) * CB, lane);
      // inputs 8 qq .. 8 qq + 7 of block kg BK + j: tile 2 (kg BK + j) + qq / 2,
      // elements 8 (qq % 2) .. + 8 of the token's 16
      const int qq = lane >> 4;
      const float* hr =
          a.hbuf + (((size_t)u * (a.hI / 16) + 2 * kg * BK + (qq >> 1)) * R + tok_a) * 16 + 8 * (qq & 1);
#pragma unroll
      for (int j = 0; j < BK; ++j) {
        hv[q][j][0] = *reinterpret_cast<const float4_t*>(hr + 2 * j * R * 16);
        hv[q][j][1] = *reinterpret_cast<const float4_t*>(hr + 2 * j * R * 16 + 4);
      }
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (!ok[q]) continue;
      // the item's scale for each token: the largest |h| of the token over
      // the item's inputs (this lane's values, then the other lanes holding
      // the same token: 8 apart, or 16 apart with 16 token rows)
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < BK; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(hv[q][j][c >> 2][c & 3]));
      if (!T16) m = fmaxf(m, __shfl_xor(m, 8, 64));
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const int eh_a = fp16_exponent_for(m);
      float4_t part[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) part[t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < BK; ++j) {
        half8_t A, Al;
        h_fragment<AM>(hv[q][j], eh_a, lane, A, Al);
        // the accumulator seed -2^(b-1) sum_k A[m][k], with the row sums laid
        // out as the accumulators by a product with an all-ones B operand
        float4_t cin = float4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (moe_code_offset(BITS) != 0) {
          cin = mfma16x16x32(A, ones, cin);
          if constexpr (AM == MOE_AM_HL16) cin = mfma16x16x32(Al, ones, cin);
          cin = off * cin;
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int f = t * BK + j;
          const half8_t B = chunk_frag<BITS>(c[q], f);
          float4_t C = mfma16x16x32(A, B, cin);
          if constexpr (AM == MOE_AM_HL16) C = mfma16x16x32(Al, B, C);
          part[t] += chunk_scale(c[q].scales, f) * C;
        }
      }
      // undo the item's scaling of the accumulator rows' tokens: 2^eh, exact
      // (lane t < 8, or < 16 with 16 token rows, holds token t's exponent)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int eh = __shfl(eh_a, tok_c + i, 64);
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t][i] += ldexpf(part[t][i], eh);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wv * RT * 4 + t * 4 + i) * 64 + lane] = acc[t][i];
  __syncthreads();
  {
    // the RT x 4 accumulator rows are shared out over the waves; each adds
    // the waves' partial sums in wave order
    const int T = a.T, d = a.d, n = lane & 15;
    for (int pi = wv; pi < RT * 4; pi += nw) {
      const int t = pi >> 2, i = pi & 3;
      float part[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) part[w] = red[((w < nw ? w : 0) * RT * 4 + pi) * 64 + lane];
      float s = part[0];
#pragma unroll
      for (int w = 1; w < 8; ++w)
        if (w < nw) s += part[w];
      if (!T16) s = add_partner32(s);  // (16 token rows: C row = token)
      const int tok = 4 * (lane >> 4) + i;  // (hi/lo: lanes < 32 hold tokens 0..7)
      const int o = rg * 16 * RT + 16 * t + n;
      if ((T16 || lane < 32) && tok < T) st_dev(a.ypart + ((size_t)sp * R + tok) * d + o, s);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial sums are stored (a signal may follow the barrier)
  __syncthreads();  // red is free again
}


}  // namespace
