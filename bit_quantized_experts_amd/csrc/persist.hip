// persist.hip -- the decode path of a whole stack of layers as one persistent
// kernel: one workgroup per CU runs, for every layer, the router role, the
// gate/up items and a down role (the same device code as the per-phase
// kernels: route_dev.h, decode_dev.h), handing results over through
// device-coherent stores and per-layer counters instead of kernel
// boundaries.  The layers of a stack are read one after another, as the
// engines on the pages read a model layer by layer [strata-mlx wiki,
// "Measured"]; a verify pass carries up to eight tokens [devlabs blog
// "32GB Mac mini 6 跑 125B 大模型", section 核心技术特点, MTP item].
//
// Dataflow of layer l (every wait is bounded, see wg_wait):
//   route   role (cs, rs): waits until the 4 S down roles that produce its
//           input columns have counted on y_ready[l-1][cs], sums their
//           partials, computes its partial logits; the last role of row
//           slice rs finishes the slice's logits and counts on logits_ready;
//   gate/up every workgroup waits for logits_ready == n_rs, selects every
//           token's experts itself (the same slot list in every workgroup),
//           runs its share of the (slot, 16-row tile) items, and counts each
//           finished item on h_ready[l][slot];
//   down    role (rg, sp): waits until every item of its slots is counted,
//           multiplies, writes its split partial and counts on
//           y_ready[l][cs] of its columns.
// The router rows of a role are loaded before its wait, so they arrive while
// the previous layer finishes.  Every layer has its own copies of the
// buffers the router step hands to the gate/up step (layer input, logits,
// divisors, exponents) and of h, so each is written once per pass and its
// many readers use L2-cached loads.  Counters sit on separate 128-byte lines.
#include "decode_dev.h"
#include "route_dev.h"

namespace {

// The down weights this workgroup's down roles will multiply depend only on
// the slot list, which every workgroup knows after its selection: one 4-byte
// load per 128-byte line brings them into the XCD's L2 while the gate/up
// items stream (the values land in the selection's scratch LDS, unused by
// then), so the down roles find them there instead of waiting for HBM.
template <int BITS, int RT>
DEVI void warm_down_weights(const PersistArgs& P, const ExpertSet& X, GuLds& L, int b, int G) {
  constexpr int CB = moe_chunk_bytes(BITS), LPC = CB / 128;
  const int tid = opaque_tid(), lane = tid & 63, wv = tid >> 6;
  const int S = P.S, n_rg = P.n_rg, base = P.has_shared ? 1 : 0;
  const int ns = base + L.S.n_routed;
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  for (int r = b; r < n_rg * S; r += G) {
    const int rg = r % n_rg, sp = r / n_rg;
    const int n_sl = sp < ns ? (ns - sp + S - 1) / S : 0;  // slots sp, sp + S, ...
    // the split's slots in order; the shared expert (slot 0) has its own k-groups
    const int n_kg0 = (sp == 0 && base) ? P.n_kg_s : P.n_kg_r;
    const int lines = n_sl > 0 ? n_kg0 * LPC + (n_sl - 1) * P.n_kg_r * LPC : 0;
    for (int i0 = wv * 64; i0 < lines; i0 += 64 * GU_NW) {
      int i = min(i0 + lane, lines - 1);
      int j = 0, nkg = n_kg0;
      if (i >= n_kg0 * LPC) {
        i -= n_kg0 * LPC;
        j = 1 + i / (P.n_kg_r * LPC);
        i -= (j - 1) * P.n_kg_r * LPC;
        nkg = P.n_kg_r;
      }
      const int u = sp + S * j, kg = i / LPC, c = i - kg * LPC;
      const uint8_t* m = (u == 0 && base) ? X.shared + X.sh_off_down
                                          : X.experts + (int64_t)L.S.expert[u] * X.ex_stride + X.off_down;
      __builtin_amdgcn_global_load_lds(m + ((int64_t)rg * nkg + kg) * CB + 128 * c, (lds_ptr_t)&L.tk_buf[wv][0], 4, 0,
                                       0);
    }
  }
}

template <int BITS, int NPER, int RT, bool A16>
__global__ __launch_bounds__(512) void decode_persist_kernel(PersistArgs P) {
  __shared__ GuLds L;
  constexpr int AM = A16 ? MOE_AM_F16 : MOE_AM_HL8;  // (16 hi/lo token rows run as per-phase kernels)
  constexpr int R = moe_am_tokens(AM);
  const int b = blockIdx.x, G = gridDim.x;
  const int T = P.T, d = P.d, n_cs = P.n_cs, n_rs = P.n_rs, S = P.S, n_rg = P.n_rg;
  const bool forced = P.in_idx != nullptr;
  const int n_rs_run = forced ? 1 : n_rs;
  const uint32_t per_cs = (uint32_t)(MOE_ROUTE_COLS / (16 * RT)) * (uint32_t)S;
  float(*ys)[MOE_ROUTE_COLS] = reinterpret_cast<float(*)[MOE_ROUTE_COLS]>(L.xs);

  constexpr int CS = MOE_CTR_STRIDE;
  for (int l = 0; l < P.n_layers; ++l) {
    const uint8_t* pb = P.base[l];
    uint32_t* ctl = P.ctl + (size_t)l * P.cpl;
    uint32_t* route_ctr = ctl;
    uint32_t* logits_ready = ctl + n_rs * CS;
    uint32_t* y_ready = ctl + (n_rs + 1) * CS;
    uint32_t* h_ready = y_ready + n_cs * CS;
    const uint32_t* y_prev = l > 0 ? P.ctl + (size_t)(l - 1) * P.cpl + (n_rs + 1) * CS : nullptr;
    float* logits = P.logits + (size_t)l * P.logits_stride;
    float* rnorm = P.rnorm + (size_t)l * MOE_PERSIST_TOK_STRIDE;
    XFrag xf;
    xf.frag = P.x.frag + (size_t)l * P.xfrag_stride;
    xf.cs = P.x.cs + (size_t)l * P.xcs_stride;
    xf.sx = P.x.sx + (size_t)l * P.xsx_stride;
    float* hbuf = P.hbuf + (size_t)l * P.hbuf_stride;

    // ---------------------------------------------------------- router ---
    RouteArgs ra{};
    ra.in = l == 0 ? P.in : P.ypart;
    ra.S_in = l == 0 ? P.S_in : S;
    ra.in_stride = l == 0 ? P.in_stride : (int64_t)R * d;
    ra.wh = reinterpret_cast<const _Float16*>(pb + P.off_wh);
    ra.wl = reinterpret_cast<const _Float16*>(pb + P.off_wl);
    ra.T = T;
    ra.d = d;
    ra.E = P.E;
    ra.code_off = P.code_off;
    ra.do_logits = !forced;
    ra.am = AM;
    ra.lp = P.lp;
    ra.x = xf;
    ra.y_out = l == 0 ? P.y_prev_out : (P.y_layers ? P.y_layers + (size_t)(l - 1) * P.yl_stride : nullptr);
    SelectArgs& sa = ra.sel;
    sa.ss_part = P.ss_part;
    sa.br = reinterpret_cast<const float*>(pb + P.off_br);
    sa.ew = reinterpret_cast<const int32_t*>(pb + P.off_ew);
    sa.n_cs = n_cs;
    sa.n_rs = n_rs_run;
    sa.T = T;
    sa.d = d;
    sa.E = P.E;
    sa.norm = l == 0 ? P.norm0 : 1;
    sa.eps = P.eps;
    sa.ctrl = route_ctr;
    sa.ctrl_stride = CS;
    sa.logits = logits;
    sa.logits_stride = P.logits_row;
    sa.rnorm = rnorm;
    sa.out_logits = (l == 0 && !forced) ? P.out_logits : nullptr;
    for (int r = b; r < n_cs * n_rs_run; r += G) {
      const int cs = r % n_cs, rs = r / n_cs;
      if (!route_role<true>(ra, cs, rs, ys, L.xe, &L.flag, y_prev ? y_prev + (size_t)cs * CS : nullptr, per_cs,
                            P.status, logits_ready))
        return;
    }

    // --------------------------------------------------------- gate/up ---
    if (!wg_wait(logits_ready, (uint32_t)n_rs_run, P.status, &L.flag)) return;
    GuArgs ga{};
    ga.X.experts = pb + P.off_ex;
    ga.X.ex_stride = P.ex_stride;
    ga.X.shared = P.has_shared ? pb + P.off_sh : nullptr;
    ga.X.off_gate = P.off_gate;
    ga.X.off_up = P.off_up;
    ga.X.off_down = P.off_down;
    ga.X.sh_off_gate = P.sh_off_gate;
    ga.X.sh_off_up = P.sh_off_up;
    ga.X.sh_off_down = P.sh_off_down;
    ga.logits = forced ? nullptr : logits;
    ga.logits_stride = P.logits_row;
    ga.idx = P.in_idx;
    ga.w = P.in_w;
    ga.out_idx = P.idx_layers ? P.idx_layers + (size_t)l * P.route_stride : nullptr;
    ga.out_w = P.w_layers ? P.w_layers + (size_t)l * P.route_stride : nullptr;
    ga.k = P.k;
    ga.rnorm = rnorm;
    ga.x = xf;
    ga.hbuf = hbuf;
    ga.E = P.E;
    ga.I = P.I;
    ga.Is = P.Is;
    ga.T = T;
    ga.d = d;
    ga.n_kg = d / 256;
    ga.bits = BITS;
    ga.hI = P.hI;
    ga.code_off = P.code_off;
    ga.has_shared = P.has_shared;
    ga.am = AM;
    gu_select<BITS, NPER, AM>(ga, L, b == 0, false);
    warm_down_weights<BITS, RT>(P, ga.X, L, b, G);
    gu_items<BITS, AM>(ga, L, b, G, h_ready);
    __syncthreads();

    // ------------------------------------------------------------ down ---
    DownArgs da{};
    da.X = ga.X;
    da.hbuf = hbuf;
    da.E = P.E;
    da.d = d;
    da.T = T;
    da.bits = BITS;
    da.hI = P.hI;
    da.BK = 8 / RT;
    da.RT = RT;
    da.n_kg_r = P.n_kg_r;
    da.n_kg_s = P.n_kg_s;
    da.S = S;
    da.has_shared = P.has_shared;
    da.max_slots = MOE_MAX_SLOTS;
    da.am = AM;
    da.ypart = P.ypart;
    const int base = P.has_shared ? 1 : 0;
    const int ns = base + L.S.n_routed;
    for (int r = b; r < n_rg * S; r += G) {
      const int rg = r % n_rg, sp = r / n_rg;
      for (int u = sp; u < ns; u += S) {
        const uint32_t tiles = (uint32_t)((u == 0 && base) ? P.Is / 16 : P.I / 16);
        if (!wg_wait(h_ready + (size_t)u * CS, tiles, P.status, &L.flag)) return;
      }
      down_role<BITS, RT, AM>(da, rg, sp, ns, L.S.expert, reinterpret_cast<float*>(L.xs));
      if (threadIdx.x == 0) {
        // every wavefront's partial sums are stored (each waited before the
        // role's last barrier)
        signal_add(y_ready + (size_t)((rg * 16 * RT) / MOE_ROUTE_COLS) * CS);
      }
    }
  }

  // ---------------------------------------------- the last layer's sum ---
  // the split partials of the last layer added in split order (as the
  // per-phase path's combine kernel does) into y and the last layer's output
  if (!P.y) return;
  const uint32_t* y_last = P.ctl + (size_t)(P.n_layers - 1) * P.cpl + (n_rs + 1) * CS;
  const __amdgpu_buffer_rsrc_t pr = coh_rsrc(P.ypart);
  for (int cs = b; cs < n_cs; cs += G) {
    if (!wg_wait(y_last + (size_t)cs * CS, per_cs, P.status, &L.flag)) return;
    for (int i = threadIdx.x; i < T * (MOE_ROUTE_COLS / 4); i += blockDim.x) {
      const int t = i / (MOE_ROUTE_COLS / 4), c = cs * MOE_ROUTE_COLS + 4 * (i % (MOE_ROUTE_COLS / 4));
      float4_t v[MOE_MAX_IN_SPLITS];
#pragma unroll
      for (int s = 0; s < MOE_MAX_IN_SPLITS; ++s)
        v[s] = coh_ld4(pr, (uint32_t)(((size_t)min(s, S - 1) * R + t) * d + c) * 4);
      float4_t acc = v[0];
#pragma unroll
      for (int s = 1; s < MOE_MAX_IN_SPLITS; ++s)
        if (s < S) acc += v[s];
      *reinterpret_cast<float4_t*>(P.y + (size_t)t * d + c) = acc;
      if (P.y_layers)
        *reinterpret_cast<float4_t*>(P.y_layers + (size_t)(P.n_layers - 1) * P.yl_stride + (size_t)t * d + c) = acc;
    }
  }
}

// Clears the per-layer counters of a pass, and the abort word.
__global__ void persist_clear_kernel(uint32_t* region, size_t n, uint32_t* status) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) region[i] = 0u;
  if (i == 0) *status = 0u;
}

template <int BITS, int NPER, bool A16>
hipError_t launch_rt(const PersistArgs& a, int rt, int grid, hipStream_t s) {
  switch (rt) {
    case 1: MOE_LAUNCH((decode_persist_kernel<BITS, NPER, 1, A16>), dim3(grid), dim3(512), 0, s, a); break;
    case 2: MOE_LAUNCH((decode_persist_kernel<BITS, NPER, 2, A16>), dim3(grid), dim3(512), 0, s, a); break;
    case 4: MOE_LAUNCH((decode_persist_kernel<BITS, NPER, 4, A16>), dim3(grid), dim3(512), 0, s, a); break;
    case 8: MOE_LAUNCH((decode_persist_kernel<BITS, NPER, 8, A16>), dim3(grid), dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS, int NPER>
hipError_t launch_a16(const PersistArgs& a, int rt, int grid, bool act16, hipStream_t s) {
  return act16 ? launch_rt<BITS, NPER, true>(a, rt, grid, s) : launch_rt<BITS, NPER, false>(a, rt, grid, s);
}

}  // namespace

bool persist_supported(int E, int bits) { return E <= 1024 && (bits == 2 || bits == 3); }

// Resident workgroups per CU of the persistent kernel: the smallest over its
// instantiations (the pass needs one per CU).
int persist_blocks_per_cu() {
  int m = 1 << 30;
  auto q = [&](const void* f) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 512, 0) != hipSuccess) n = 0;
    m = n < m ? n : m;
  };
#define PQ(B, N, R, A) q(reinterpret_cast<const void*>(&decode_persist_kernel<B, N, R, A>))
#define PQ4(B, N, A) PQ(B, N, 1, A); PQ(B, N, 2, A); PQ(B, N, 4, A); PQ(B, N, 8, A)
  PQ4(2, 8, false); PQ4(2, 16, false); PQ4(3, 8, false); PQ4(3, 16, false);
  PQ4(2, 8, true); PQ4(2, 16, true); PQ4(3, 8, true); PQ4(3, 16, true);
#undef PQ4
#undef PQ
  return m;
}

hipError_t launch_persist(const PersistArgs& a, int rt, int grid, bool act16, size_t clear_words, hipStream_t s) {
  if (clear_words) {
    hipLaunchKernelGGL(persist_clear_kernel, dim3((unsigned)((clear_words + 255) / 256)), dim3(256), 0, s, a.ctl,
                       clear_words, a.status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool small = a.E <= 512;
  if (a.bits == 2) return small ? launch_a16<2, 8>(a, rt, grid, act16, s) : launch_a16<2, 16>(a, rt, grid, act16, s);
  return small ? launch_a16<3, 8>(a, rt, grid, act16, s) : launch_a16<3, 16>(a, rt, grid, act16, s);
}
