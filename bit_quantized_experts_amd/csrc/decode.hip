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
// Memory: weight chunks stream from HBM into registers, several k-groups
// ahead of the multiplies; the gate/up activation fragments are read from
// LDS (one copy per workgroup), the down kernel's h fragments from L2.
#include "kern_common.h"
#include "moe_launch.h"
#include "topk.h"

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

// A-fragment and accumulator seed of block b of the h fragments: the seed is
// the sum of the two 16-row tile sums the gate/up kernel wrote for the block.
DEVI void load_a(const _Float16* frag, const float* sum, size_t b, int lane, half8_t& A, float4_t& cin) {
  A = *reinterpret_cast<const half8_t*>(frag + (b * 64 + lane) * 8);
  const float4_t c0 = *reinterpret_cast<const float4_t*>(sum + (2 * b) * 16 + 4 * (lane >> 4));
  const float4_t c1 = *reinterpret_cast<const float4_t*>(sum + (2 * b + 1) * 16 + 4 * (lane >> 4));
  cin = c0 + c1;
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
  const int lane = threadIdx.x & 63;
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
// Inputs wider than GU_WIN blocks are staged in windows, one after another.
// ---------------------------------------------------------------------------
constexpr int GU_NW = 8;    // wavefronts per workgroup
constexpr int GU_WIN = 96;  // activation blocks staged in LDS at once

struct alignas(16) GuLds {
  alignas(16) unsigned char xs[GU_WIN * 1024];  // A-fragments, [block][lane][8] fp16
  alignas(16) float cs[GU_WIN * 16];  // accumulator seeds, [block][16]
  float red[GU_NW][8][64];          // partial sums of the k-parts
  float rn[16];                     // 1 / rms of each token
  SlotLds S;
  uint64_t tk_buf[GU_NW][TOPK_BUF];
};

template <int BITS>
struct GroupRegs {
  ChunkRegs<BITS> g, u;
};

// Activation blocks [b0, b0 + nblk) into LDS (plain loads and LDS stores),
// in two halves so that other work can run while the loads are in flight.
// Entry p of a block is lane p % 64 of its A-fragment, which holds token
// (p % 64) & 7 (fp16 activations: (p % 64) & 15); the rows of tokens >= T are
// zeros (as the route kernel writes them), so they are stored without being
// read.
struct WindowRegs {
  static constexpr int PER = GU_WIN * 64 / (64 * GU_NW);
  u32x4_t v[PER];
  float4_t c;
};

DEVI void window_load(WindowRegs& W, const GuArgs& a, int b0, int nblk, int tid) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.xfrag + (size_t)b0 * 512);
  const int n = nblk * 64, nc = nblk * 4;
  const bool live = (tid & (a.act16 ? 15 : 7)) < a.T;  // (64 * GU_NW is a multiple of 64: same lane for every i)
#pragma unroll
  for (int i = 0; i < WindowRegs::PER; ++i) {
    const int p = tid + 64 * GU_NW * i;
    W.v[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (p < n && live) W.v[i] = src[p];
  }
  W.c = float4_t{0.f, 0.f, 0.f, 0.f};
  if (tid < nc) W.c = reinterpret_cast<const float4_t*>(a.xsum + (size_t)b0 * 16)[tid];
}

DEVI void window_store(const WindowRegs& W, GuLds& L, int nblk, int tid) {
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(L.xs);
  const int n = nblk * 64, nc = nblk * 4;
#pragma unroll
  for (int i = 0; i < WindowRegs::PER; ++i) {
    const int p = tid + 64 * GU_NW * i;
    if (p < n) dst[p] = W.v[i];
  }
  if (tid < nc) reinterpret_cast<float4_t*>(L.cs)[tid] = W.c;
}

DEVI void stage_window(GuLds& L, const GuArgs& a, int b0, int nblk, int tid) {
  WindowRegs W;
  window_load(W, a, b0, nblk, tid);
  window_store(W, L, nblk, tid);
}

template <int BITS>
DEVI void issue_group(GroupRegs<BITS>& r, const uint8_t* gate, const uint8_t* up, int64_t off, int lane) {
  load_chunk<BITS>(r.g, gate + off, lane);
  load_chunk<BITS>(r.u, up + off, lane);
}

// Eight blocks (one k-group) of gate and up; lb = first block in the window.
template <int BITS>
DEVI void mul_group(const GroupRegs<BITS>& r, const GuLds& L, int lb, int lane, float4_t& accg, float4_t& accu) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const half8_t A = *reinterpret_cast<const half8_t*>(L.xs + (size_t)(lb + j) * 1024 + 16 * lane);
    const float4_t cin = *reinterpret_cast<const float4_t*>(L.cs + (lb + j) * 16 + 4 * (lane >> 4));
    const float4_t Cg = mfma16x16x32(A, chunk_frag<BITS>(r.g, j), cin);
    const float4_t Cu = mfma16x16x32(A, chunk_frag<BITS>(r.u, j), cin);
    accg += chunk_scale(r.g.scales, j) * Cg;
    accu += chunk_scale(r.u.scales, j) * Cu;
  }
}

// k-groups kg0, kg0 + step, ... below kg1 of one 16-row tile (chunk row
// offset rowoff); the window starts at k-group wkg0.  A three-slot register
// ring: each step of the main loop issues the k-group two steps ahead (the
// last k-group again once past the end) and multiplies the oldest one; the
// main loop has no early exit, so the loads in flight at every multiply are
// the same and the compiler's wait counts stay exact; a tail of up to two
// steps multiplies what is already in flight.
template <int BITS>
DEVI void run_tile(const uint8_t* gate, const uint8_t* up, int64_t rowoff, int kg0, int kg1, int step, int wkg0,
                   const GuLds& L, int lane, float4_t& accg, float4_t& accu) {
  constexpr int64_t CB = BITS == 2 ? 1280 : 1792;
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
    mul_group<BITS>(r0, L, 8 * (kg - wkg0), lane, accg, accu);
    kg += step;
    issue_group<BITS>(r0, gate, up, rowoff + min(kg + 2 * step, last) * CB, lane);
    __builtin_amdgcn_sched_barrier(0);
    mul_group<BITS>(r1, L, 8 * (kg - wkg0), lane, accg, accu);
    kg += step;
    issue_group<BITS>(r1, gate, up, rowoff + min(kg + 2 * step, last) * CB, lane);
    __builtin_amdgcn_sched_barrier(0);
    mul_group<BITS>(r2, L, 8 * (kg - wkg0), lane, accg, accu);
    kg += step;
  }
  const int rem = nsteps % 3;
  if (rem >= 1) mul_group<BITS>(r0, L, 8 * (kg - wkg0), lane, accg, accu);
  if (rem == 2) mul_group<BITS>(r1, L, 8 * (kg + step - wkg0), lane, accg, accu);
}

template <int BITS, int NPER>  // NPER >= ceil(E / 64)
__global__ __launch_bounds__(64 * GU_NW) void gu_decode_kernel(GuArgs a) {
  constexpr int64_t CB = BITS == 2 ? 1280 : 1792;
  __shared__ GuLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: loop bounds stay scalar
  const int T = a.T, k = a.k, E = a.E, tk = a.T * a.k;
  const bool has_shared = a.has_shared != 0;
  const int base = has_shared ? 1 : 0;
  const int tiles_r = a.I / 16, tiles_s = has_shared ? a.Is / 16 : 0;
  const int n_kg = a.n_kg;
  const int n_win = (8 * n_kg + GU_WIN - 1) / GU_WIN;
  const int win_kg = (n_kg + n_win - 1) / n_win;  // k-groups per window

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
      const float* row = a.logits + (size_t)min(wv + GU_NW * h, T - 1) * E;
#pragma unroll
      for (int i = 0; i < NPER; ++i) lv[h][i] = row[min(lane + 64 * i, E - 1)];
    }
  }
  const float rnv = (tid >= 64 && tid < 64 + T) ? a.rnorm[tid - 64] : 1.0f;
  // the activation window (one window for inputs of up to GU_WIN blocks)
  // stays in registers through the selection and is stored to LDS before the
  // barrier that ends it: the selection starts as soon as its logits are in,
  // while the larger window is still arriving
  WindowRegs win;
  if (n_win == 1) window_load(win, a, 0, 8 * n_kg, tid);
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
          const float* row = a.logits + (size_t)t * E;
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
  if (n_win == 1) window_store(win, L, 8 * n_kg, tid);
  if (tid >= 64 && tid < 80) L.rn[tid - 64] = 1.0f / rnv;
  lds_barrier();  // every token's experts marked, the window staged
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wv + GU_NW * h;
    if (t < T) {
      place_lane<NPER>(L.S, mine[h].e, mine[h].w, t, k, E, base, !select, t == 0);
      if (blockIdx.x == 0 && lane < k) {  // the routing used (given rows are copied as they are)
        if (a.out_idx) a.out_idx[t * k + lane] = mine[h].e;
        if (a.out_w) a.out_w[t * k + lane] = mine[h].w;
      }
    }
  }
  lds_barrier();  // slot list, rms and the staged activations
  if (blockIdx.x == 0) {
    const int ns = base + L.S.n_routed;
    if (tid == 0) *a.n_slots = ns;
    for (int i = tid; i < ns; i += blockDim.x) a.slot_expert[i] = L.S.expert[i];
    for (int i = tid; i < ns * 16; i += blockDim.x) a.slot_w[i] = L.S.w[i >> 4][i & 15];
  }
  const int n_items = tiles_s + L.S.n_routed * tiles_r;
  int KP = 8;
  while (KP > 1 && (KP > n_kg || n_items * KP > (int)gridDim.x * GU_NW)) KP >>= 1;
  const int G = GU_NW / KP, jw = wv / KP, kp = wv - jw * KP;
  const int tok_e = 4 * ((lane >> 4) & 1);

  for (int grp = blockIdx.x; grp * G < n_items; grp += gridDim.x) {
    const int item = grp * G + jw;
    const bool valid = item < n_items;
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
    for (int w = 0; w < n_win; ++w) {
      const int kg0 = w * win_kg, kg1 = min(n_kg, kg0 + win_kg);
      if (n_win > 1) {
        __syncthreads();
        stage_window(L, a, 8 * kg0, 8 * (kg1 - kg0), tid);
        __syncthreads();
      }
      if (valid) run_tile<BITS>(gate, up, (int64_t)t * n_kg * CB, kg0 + kp, kg1, KP, kg0, L, lane, accg, accu);
    }
    if (KP > 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L.red[wv][i][lane] = accg[i];
        L.red[wv][4 + i][lane] = accu[i];
      }
      __syncthreads();
      if (kp == 0) {
        for (int p = 1; p < KP; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accg[i] += L.red[wv + p][i][lane];
            accu[i] += L.red[wv + p][4 + i][lane];
          }
      }
    }
    if (valid && kp == 0) {
      // lane l: intermediate row n = l & 15 of the tile, C rows 4(l>>4)+i:
      // tokens tok_e + i, hi part in lanes < 32, lo part in lanes >= 32 (fp16
      // activations: token 4(l>>4)+i, no lo part)
      const int n = lane & 15;
      const bool a16 = a.act16 != 0;
      const bool lo_half = !a16 && lane >= 32;
      const int pblk = t >> 1, kk = 16 * (t & 1) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = a16 ? 4 * (lane >> 4) + i : tok_e + i;
        const float gw = (u == 0 && has_shared) ? (tok < T ? 1.0f : 0.f) : L.S.w[u][tok];
        const float rrn = L.rn[tok];  // 1 / rms
        const float g = (a16 ? accg[i] : add_partner32(accg[i])) * rrn;
        const float uu = (a16 ? accu[i] : add_partner32(accu[i])) * rrn;
        const float hv = g * __builtin_amdgcn_rcpf(1.0f + expf(-g)) * uu;
        const float hs = (gw != 0.f) ? gw * hv : 0.f;
        const _Float16 hi = (_Float16)hs;
        const _Float16 val = lo_half ? (_Float16)(hs - (float)hi) : hi;
        const int mrow = a16 ? tok : tok + (lo_half ? 8 : 0);
        a.hfrag[(((size_t)u * a.nbI + pblk) * 64 + mrow + 16 * (kk >> 3)) * 8 + (kk & 7)] = val;
        const float sm = row16_sum((float)val);
        if (n == 0) a.hsum[((size_t)u * 2 * a.nbI + t) * 16 + mrow] = -(float)a.code_off * sm;
      }
    }
    if (KP > 1) __syncthreads();  // red is rewritten in the next round
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
    pre0 = a.slot_expert[min(u0, a.max_slots - 1)];
    pre1 = a.slot_expert[min(u1, a.max_slots - 1)];
  }
  const int n_rs = (first_r < ns) ? (ns - first_r + S - 1) / S : 0;
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
        int e = (b0 == wv) ? ((ok[q] && q == 1) ? pre1 : pre0) : a.slot_expert[u];
        e = min(max(e, 0), a.E - 1);
        mat = a.X.experts + (int64_t)e * a.X.ex_stride + a.X.off_down;
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
      const bool a16 = a.act16 != 0;  // fp16 activations: C row = token, 16 tokens
      if (!a16) s = add_partner32(s);
      const int tok = 4 * (lane >> 4) + i;  // (hi/lo: lanes < 32 hold tokens 0..7)
      const int o = rg * 16 * RT + 16 * t + n;
      if ((a16 || lane < 32) && tok < T) a.ypart[((size_t)sp * (a16 ? 16 : 8) + tok) * d + o] = s;
    }
}

template <int BITS, int RT>
hipError_t launch_down_t(const DownArgs& a, int grid_x, int nw, hipStream_t s) {
  MOE_LAUNCH((down_decode_kernel<BITS, RT>), dim3(grid_x, a.S), dim3(64 * nw), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gu_decode(const GuArgs& a, int n_wg, hipStream_t s) {
#define GU_LAUNCH(B, N) MOE_LAUNCH((gu_decode_kernel<B, N>), dim3(n_wg), dim3(64 * GU_NW), 0, s, a)
  const int np = a.E <= 512 ? 8 : a.E <= 1024 ? 16 : a.E <= 2048 ? 32 : 64;
  if (a.bits == 2) {
    if (np == 8) GU_LAUNCH(2, 8);
    else if (np == 16) GU_LAUNCH(2, 16);
    else if (np == 32) GU_LAUNCH(2, 32);
    else GU_LAUNCH(2, 64);
  } else {
    if (np == 8) GU_LAUNCH(3, 8);
    else if (np == 16) GU_LAUNCH(3, 16);
    else if (np == 32) GU_LAUNCH(3, 32);
    else GU_LAUNCH(3, 64);
  }
#undef GU_LAUNCH
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
