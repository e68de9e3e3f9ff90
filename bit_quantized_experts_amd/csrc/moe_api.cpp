// moe_api.cpp -- the C ABI declared in include/moe.h: argument checks, the
// packed and workspace layouts, and the order of kernel launches.  No device
// memory is allocated here; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"
#include "moe_launch.h"

thread_local MoeLaunchEvents moe_launch_events;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

// Compute units of the current device (cached per device id).
int cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Workgroups of a persistent pass: one per CU, all resident at once (the
// kernel's waits need every workgroup running); 0 if the kernel cannot hold
// one workgroup per CU on this device.
int persist_grid() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) cached[dev] = persist_blocks_per_cu() >= 1 ? cu_count() : -1;
  return cached[dev] > 0 ? cached[dev] : 0;
}

std::once_flag g_init_once;
hipError_t g_init_err = hipSuccess;
void init_kernels() {
  std::call_once(g_init_once, [] { g_init_err = moe_route_kernels_init(); });
}

int choose_bk(int nb) {
  for (int bk : {8, 4, 2, 1})
    if (nb % bk == 0) return bk;
  return 1;
}

bool make_mat(int rows, int cols, int bits, moe_mat_layout* L, int bk = 0) {
  L->rows = rows;
  L->cols = cols;
  L->nb = cols / 32;
  L->BK = bk > 0 ? bk : choose_bk(L->nb);
  if (L->nb % L->BK) return false;
  L->RT = 8 / L->BK;
  if (rows % (16 * L->RT) != 0) return false;
  L->n_rg = rows / (16 * L->RT);
  L->n_kg = L->nb / L->BK;
  L->chunk_bytes = moe_chunk_bytes(bits);
  L->bytes = (int64_t)L->n_rg * L->n_kg * L->chunk_bytes;
  return true;
}

// Down matrices of the routed and the shared expert share one block grouping
// (the largest power of two <= 8 dividing both d_ff/32 and d_ff_shared/32),
// so a row group of the down kernel has the same height for every expert.
int down_bk(int I, int Is) {
  int a = I / 32, b = Is > 0 ? Is / 32 : a;
  while (b) { int t = a % b; a = b; b = t; }
  return choose_bk(a);
}

bool make_expert(int d, int I, int bits, moe_expert_layout* X, int bk_down) {
  if (!make_mat(I, d, bits, &X->gate) || !make_mat(I, d, bits, &X->up) || !make_mat(d, I, bits, &X->down, bk_down))
    return false;
  X->off_gate = 0;
  X->off_up = moe_align256(X->gate.bytes);
  X->off_down = X->off_up + moe_align256(X->up.bytes);
  X->bytes = moe_align256(X->off_down + X->down.bytes);
  return true;
}

// Canonical bytes of one block of a kind (2, 3: b-bit codes; codebook: 15).
int64_t canon_block_bytes(int kind) { return kind == MOE_KIND_CB ? 15 : 2 + 4 * kind; }

// The kernels' block kind of a descriptor (the layer keeps it in `bits`).
int desc_kind(const moe_layer_desc* D) { return D->codebook ? MOE_KIND_CB : D->bits; }

int check_desc(const moe_layer_desc* D) {
  if (!D) return fail(MOE_ERR_ARG, "desc is NULL");
  if (D->block != 32) return fail(MOE_ERR_UNSUPPORTED, "block must be 32 (got %d)", D->block);
  if (D->bits != 2 && D->bits != 3) return fail(MOE_ERR_UNSUPPORTED, "bits must be 2 or 3 (got %d)", D->bits);
  if (D->codebook != 0 && D->codebook != 1) return fail(MOE_ERR_ARG, "codebook must be 0 or 1 (got %d)", D->codebook);
  if (D->codebook && D->bits != 3)
    return fail(MOE_ERR_UNSUPPORTED, "codebook blocks are of the 3-bit class: bits must be 3 (got %d)", D->bits);
  if (D->d_model <= 0 || D->d_model % 256) return fail(MOE_ERR_UNSUPPORTED, "d_model must be a positive multiple of 256 (got %d)", D->d_model);
  if (D->d_model > 8192) return fail(MOE_ERR_UNSUPPORTED, "d_model above 8192 not supported (got %d)", D->d_model);
  if (D->n_experts < 1 || D->n_experts > MOE_MAX_E) return fail(MOE_ERR_UNSUPPORTED, "n_experts must be in [1, %d] (got %d)", MOE_MAX_E, D->n_experts);
  if (D->d_ff <= 0 || D->d_ff % 32) return fail(MOE_ERR_UNSUPPORTED, "d_ff must be a positive multiple of 32 (got %d)", D->d_ff);
  if (D->d_ff_shared < 0 || D->d_ff_shared % 32) return fail(MOE_ERR_UNSUPPORTED, "d_ff_shared must be 0 or a multiple of 32 (got %d)", D->d_ff_shared);
  if (D->top_k < 1 || D->top_k > D->n_experts || D->top_k > MOE_MAX_K)
    return fail(MOE_ERR_ARG, "top_k must be in [1, min(n_experts, %d)] (got %d)", MOE_MAX_K, D->top_k);
  return MOE_OK;
}

// packed buffer: [status 256 B][router_w][router_b][router hi][router lo]
// [router exponents][bounds][codebook grid (codebook blocks)][E experts][shared]
struct PackedLayout {
  int64_t off_status, off_rw, off_rb, off_rwh, off_rwl, off_rew, off_hb, off_grid, off_ex, off_sh, total;
};

int e16_of(int E) { return (E + 15) / 16 * 16; }

PackedLayout packed_layout(const moe_layer_desc* D, const moe_expert_layout& ex, const moe_expert_layout& sh) {
  PackedLayout P;
  const int64_t E16 = e16_of(D->n_experts);
  P.off_status = 0;
  P.off_rw = 256;
  P.off_rb = P.off_rw + moe_align256((int64_t)D->n_experts * D->d_model * 4);
  P.off_rwh = P.off_rb + moe_align256((int64_t)D->n_experts * 4);
  P.off_rwl = P.off_rwh + moe_align256(E16 * D->d_model * 2);
  P.off_rew = P.off_rwl + moe_align256(E16 * D->d_model * 2);
  P.off_hb = P.off_rew + moe_align256(E16 * 4);
  P.off_grid = P.off_hb + moe_align256((int64_t)(D->n_experts + 1) * 8);  // hb then ed
  P.off_ex = P.off_grid + (D->codebook ? 512 * 4 * 2 : 0);
  P.off_sh = P.off_ex + (int64_t)D->n_experts * ex.bytes;
  P.total = P.off_sh + (D->d_ff_shared > 0 ? sh.bytes : 0);
  return P;
}

// ------------------------------------------------------------- workspace ---
struct WsLayout {
  int64_t ctrl, lp, ss_part, rnorm, logits, n_slots, slot_expert, slot_w, xfrag, xcs, xsx, hbuf, ypart,
      total;
  int max_slots, S, nbI, n_cs;
};

// control region: the per-phase route kernel's counters (MOE_CTRL_WORDS
// words), then the persistent pass's abort word at byte 256
int64_t ctrl_bytes() { return 512; }

// Row stride of the workspace logits: E rounded up to 64, so the 64 logits a
// row slice finishes fill cache lines no other workgroup writes.
int logits_row(int E) { return (E + 63) / 64 * 64; }
constexpr int64_t kStatusOffset = 256;

int down_splits(const moe_layer* L, int max_slots) {
  const int n_rg = L->ex.down.n_rg;
  // the down kernel's workgroups (512 threads) fit two per CU: one round of
  // n_rg * S workgroups when S = 2 CUs / n_rg
  int S = env_int("MOE_DOWN_SPLITS", 0);
  if (S <= 0) S = (2 * cu_count()) / n_rg;
  if (S > max_slots) S = max_slots;
  if (S > MOE_MAX_IN_SPLITS) S = MOE_MAX_IN_SPLITS;
  if (S < 1) S = 1;
  return S;
}

// Decode pass of T tokens; am: the activation rows (MOE_AM_*: 8 tokens hi +
// lo, 16 in fp16, 16 hi + lo).
WsLayout ws_layout_decode(const moe_layer* L, int T, int am = MOE_AM_HL8) {
  WsLayout W{};
  const int k = L->k, E = L->E, d = L->d;
  W.max_slots = (T * k < E ? T * k : E) + (L->Is > 0 ? 1 : 0);
  W.nbI = (L->I > L->Is ? L->I : L->Is) / 32;
  W.S = down_splits(L, W.max_slots);
  W.n_cs = d / MOE_ROUTE_COLS;
  int64_t o = 0;
  auto take = [&](int64_t bytes) { int64_t r = o; o += moe_align256(bytes); return r; };
  W.ctrl = take(ctrl_bytes());
  // The down partials come right after the control words, sized for the
  // most splits and rows whatever the layer's shapes: in a stack, layer l+1
  // reads layer l's partials while it writes the rest of this layout for its
  // own shapes, so their place must not depend on E, k or the expert sizes.
  W.ypart = take((int64_t)MOE_MAX_IN_SPLITS * MOE_MAX_TOK_F16ACT * d * 4);
  W.lp = take((int64_t)W.n_cs * T * E * 4);
  W.ss_part = take((int64_t)((E + MOE_ROUTE_ROWS - 1) / MOE_ROUTE_ROWS) * W.n_cs * T * 4);
  W.rnorm = take(16 * 4);
  W.logits = take((int64_t)T * logits_row(E) * 4);
  W.n_slots = take(4);
  W.slot_expert = take((int64_t)W.max_slots * 4);
  W.slot_w = take((int64_t)W.max_slots * 16 * 4);
  W.xfrag = take((int64_t)(d / 32) * moe_am_tiles(am) * 1024);
  W.xcs = take((int64_t)(d / 32) * 16 * 4);
  W.xsx = take((int64_t)W.n_cs * MOE_XSX_STRIDE * 4);
  const int R = moe_am_tokens(am);
  W.hbuf = take((int64_t)W.max_slots * R * W.nbI * 32 * 4);
  W.total = o;
  return W;
}

// Persistent decode pass of T tokens over up to n layers per launch
// (persist.hip): the router's partial results, each layer's own copies of the
// buffers the router step hands to the gate/up step and of h, and per-layer
// counters (cleared before each launch).  The down partials sit where the
// per-phase layout has them.
struct PsLayout {
  int64_t ctrl, ypart, lp, ss_part, rnorm, logits, xfrag, xcs, xsx, hbuf, ctl, total;
  int64_t logits_stride, hbuf_stride, xcs_stride, xsx_stride;  // elements per layer
  int64_t xfrag_stride;                                        // fp16 elements per layer
  int max_slots, S, n_rs, n_cs, cpl, hI;
  size_t clear_words;  // ctl
};

int persist_grid();  // workgroups of a persistent pass (0: not available)

int persist_splits(const moe_layer* L, int max_slots) {
  int S = persist_grid() / L->ex.down.n_rg;
  if (S > max_slots) S = max_slots;
  if (S > MOE_MAX_IN_SPLITS) S = MOE_MAX_IN_SPLITS;
  if (S < 1) S = 1;
  return S;
}

PsLayout ws_layout_persist(const moe_layer* L, int T, bool act16, int n_layers) {
  PsLayout W{};
  const int n = n_layers < MOE_PERSIST_MAX_LAYERS ? (n_layers < 1 ? 1 : n_layers) : MOE_PERSIST_MAX_LAYERS;
  const int R = act16 ? MOE_MAX_TOK_F16ACT : MOE_MAX_TOK_DECODE;
  const int k = L->k, E = L->E, d = L->d;
  W.max_slots = (T * k < E ? T * k : E) + (L->Is > 0 ? 1 : 0);
  W.hI = ((L->I > L->Is ? L->I : L->Is) / 32) * 32;
  W.S = persist_splits(L, W.max_slots);
  W.n_cs = d / MOE_ROUTE_COLS;
  W.n_rs = (E + MOE_ROUTE_ROWS - 1) / MOE_ROUTE_ROWS;
  W.cpl = (W.n_rs + 1 + W.n_cs + W.max_slots) * MOE_CTR_STRIDE;
  W.logits_stride = moe_align256((int64_t)T * logits_row(E) * 4) / 4;
  W.hbuf_stride = moe_align256((int64_t)W.max_slots * R * W.hI * 4) / 4;
  W.xfrag_stride = moe_align256((int64_t)(d / 32) * 1024) / 2;
  W.xcs_stride = moe_align256((int64_t)(d / 32) * 16 * 4) / 4;
  W.xsx_stride = moe_align256((int64_t)W.n_cs * MOE_XSX_STRIDE * 4) / 4;
  int64_t o = 0;
  auto take = [&](int64_t bytes) { int64_t r = o; o += moe_align256(bytes); return r; };
  W.ctrl = take(ctrl_bytes());
  W.ypart = take((int64_t)MOE_MAX_IN_SPLITS * MOE_MAX_TOK_F16ACT * d * 4);
  W.lp = take((int64_t)W.n_cs * T * E * 4);
  W.ss_part = take((int64_t)W.n_rs * W.n_cs * T * 4);
  W.rnorm = take((int64_t)n * MOE_PERSIST_TOK_STRIDE * 4);
  W.logits = take((int64_t)n * W.logits_stride * 4);
  W.xfrag = take((int64_t)n * W.xfrag_stride * 2);
  W.xcs = take((int64_t)n * W.xcs_stride * 4);
  W.xsx = take((int64_t)n * W.xsx_stride * 4);
  W.hbuf = take((int64_t)n * W.hbuf_stride * 4);
  const int64_t ctl_bytes = (int64_t)n * W.cpl * 4;
  W.ctl = take(ctl_bytes);
  W.total = o;
  W.clear_words = (size_t)ctl_bytes / 4;
  return W;
}

// Prefill workspace (T > 8).  Rows: the routed pairs grouped by expert, each
// expert padded to a multiple of 16, then one row per token for the shared
// expert (padded to 16).
struct PfLayout {
  int64_t ctrl, ex, xh, xl, logits, rpart, idx, w, tile_bm, tile_cnt, counts, offsets, n_items, item_group, item_row0,
      item_rows, row_src, row_tok, row_w, slot_pos, hfrag, ypart, rowf, total;
  int n_tiles, R, max_items, nbH, n_nt;
};

int64_t routed_rows_max(int64_t T, int k, int E) {
  const int64_t pairs = T * k;
  return pairs + 15 * (pairs < E ? pairs : E);
}

// The prefill router GEMM has one workgroup per 128 tokens x 128 experts,
// each over the whole input; with few of them (short chunks) it runs one
// workgroup per 256-column slice as well and adds the slices in a second
// kernel (same bits either way).
bool router_split(const moe_layer* L, int T) {
  const int n_tt = (T + 127) / 128, n_ey = (L->E16 + PF_ET - 1) / PF_ET;
  return n_tt * n_ey <= 64;
}

PfLayout ws_layout_prefill(const moe_layer* L, int T) {
  PfLayout W{};
  const int k = L->k, E = L->E, d = L->d;
  const int Imax = L->I > L->Is ? L->I : L->Is;
  const int64_t rr = routed_rows_max(T, k, E);
  const int64_t rs = L->Is > 0 ? (T + 15) / 16 * 16 : 0;
  const int64_t pairs = (int64_t)T * k;
  W.n_tiles = (T + PF_T64 - 1) / PF_T64;
  W.R = (int)(rr + rs);
  W.max_items = (int)((rr + PF_TM - 1) / PF_TM + (pairs < E ? pairs : E) + (rs + PF_TM - 1) / PF_TM);
  W.nbH = Imax / 32;
  W.n_nt = (Imax + PF_HT - 1) / PF_HT;
  int64_t o = 0;
  auto take = [&](int64_t bytes) { int64_t r = o; o += moe_align256(bytes); return r; };
  W.ctrl = take(ctrl_bytes());
  W.ex = take((int64_t)T * 4);
  W.xh = take((int64_t)T * d * 2);
  W.xl = take((int64_t)T * d * 2);
  W.logits = take((int64_t)T * E * 4);
  W.rpart = take(router_split(L, T) ? (int64_t)(d / 256) * T * E * 4 : 0);
  W.idx = take(pairs * 4);
  W.w = take(pairs * 4);
  W.tile_bm = take((int64_t)W.n_tiles * E * 8);
  W.tile_cnt = take((int64_t)W.n_tiles * E * 4);
  W.counts = take((int64_t)E * 4);
  W.offsets = take((int64_t)(E + 2) * 4);
  W.n_items = take(4);
  W.item_group = take((int64_t)W.max_items * 4);
  W.item_row0 = take((int64_t)W.max_items * 4);
  W.item_rows = take((int64_t)W.max_items * 4);
  W.row_src = take((int64_t)W.R * 4);
  W.row_tok = take((int64_t)W.R * 4);
  W.row_w = take((int64_t)W.R * 4);
  W.slot_pos = take(pairs * 4);
  W.hfrag = take((int64_t)W.R * Imax * 2);
  W.ypart = take((int64_t)W.R * d * 2);  // fp16 down rows
  W.rowf = take((int64_t)W.R * 4);
  W.total = o;
  return W;
}

// ---------------------------------------------------------------- timing ---
struct Timing {
  std::mutex mu;
  std::atomic<int> cls{-1};
  int max = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;
} g_timing;

// While per-kernel timing is enabled every launch of the layer functions
// waits for the stream to drain, so each kernel runs alone (events and
// profiler time stamps then cover one kernel each).
void serial_point(hipStream_t s) {
  if (g_timing.cls >= 0) hipStreamSynchronize(s);
}

// The timed launch records its own start and stop events (the dispatch's
// time stamps), so no marker sits between it and the preceding kernel.
void timed_begin(int cls, hipStream_t s, int* slot) {
  (void)s;
  *slot = -1;
  if (g_timing.cls != cls) return;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.cls != cls || g_timing.used >= g_timing.max) return;
  *slot = g_timing.used++;
  moe_launch_events.start = g_timing.ev[2 * *slot];
  moe_launch_events.stop = g_timing.ev[2 * *slot + 1];
}
void timed_end(int slot, hipStream_t s) {
  (void)slot;
  (void)s;
  moe_launch_events = MoeLaunchEvents{};
}

ExpertSet expert_set(const moe_layer* L) {
  ExpertSet X;
  X.experts = L->experts;
  X.ex_stride = L->ex.bytes;
  X.shared = L->shared;
  X.off_gate = L->ex.off_gate;
  X.off_up = L->ex.off_up;
  X.off_down = L->ex.off_down;
  X.sh_off_gate = L->sh.off_gate;
  X.sh_off_up = L->sh.off_up;
  X.sh_off_down = L->sh.off_down;
  X.grid16 = L->grid16;
  return X;
}

// Input of a decode layer: the caller's x (S = 1) or the previous layer's
// down partials in the workspace (S splits, RMSNorm applied).
struct LayerInput {
  const float* p;
  int S;
  int64_t stride;
  int norm;
};

// One decode layer (T <= moe_am_tokens(am)): route (router logits) -> gate/up
// (with the top-k selection in every workgroup) -> down.  The result
// is left as split partials in the workspace (ypart, W.S splits).
int decode_layer(const moe_layer* L, const LayerInput& in, float eps, int T, float* y_prev_out,
                 const moe_route_io* r, uint8_t* ws, hipStream_t s, int* S_out, int am = MOE_AM_HL8) {
  const WsLayout W = ws_layout_decode(L, T, am);
  const int d = L->d, E = L->E;
  const bool forced = r && r->in_idx && r->in_w;
  int slot;

  RouteArgs ra{};
  ra.in = in.p;
  ra.S_in = in.S;
  ra.in_stride = in.stride;
  ra.wh = L->router_wh;
  ra.wl = L->router_wl;
  ra.T = T;
  ra.d = d;
  ra.E = E;
  ra.code_off = moe_code_offset(L->bits);
  ra.do_logits = !forced;
  ra.am = am;
  ra.lp = reinterpret_cast<float*>(ws + W.lp);
  ra.x.frag = reinterpret_cast<_Float16*>(ws + W.xfrag);
  ra.x.cs = reinterpret_cast<float*>(ws + W.xcs);
  ra.x.sx = reinterpret_cast<int32_t*>(ws + W.xsx);
  ra.y_out = y_prev_out;
  SelectArgs& sa = ra.sel;
  sa.ss_part = reinterpret_cast<float*>(ws + W.ss_part);
  sa.br = L->router_b;
  sa.ew = L->router_ew;
  sa.n_cs = W.n_cs;
  sa.n_rs = forced ? 1 : (E + MOE_ROUTE_ROWS - 1) / MOE_ROUTE_ROWS;
  sa.T = T;
  sa.d = d;
  sa.E = E;
  sa.norm = in.norm;
  sa.eps = eps;
  sa.ctrl = reinterpret_cast<uint32_t*>(ws + W.ctrl);
  sa.ctrl_stride = 1;
  sa.logits = reinterpret_cast<float*>(ws + W.logits);
  sa.logits_stride = logits_row(E);
  sa.rnorm = reinterpret_cast<float*>(ws + W.rnorm);
  sa.out_logits = (r && !forced) ? r->out_logits : nullptr;
  timed_begin(2, s, &slot);
  serial_point(s);
  HIPCHK(launch_route(ra, s));
  timed_end(slot, s);

  const ExpertSet X = expert_set(L);
  GuArgs ga{};
  ga.X = X;
  ga.logits = forced ? nullptr : sa.logits;
  ga.logits_stride = sa.logits_stride;
  ga.idx = forced ? r->in_idx : nullptr;
  ga.w = forced ? r->in_w : nullptr;
  ga.out_idx = r ? r->out_idx : nullptr;
  ga.out_w = r ? r->out_w : nullptr;
  ga.k = L->k;
  ga.n_slots = reinterpret_cast<int32_t*>(ws + W.n_slots);
  ga.slot_expert = reinterpret_cast<int32_t*>(ws + W.slot_expert);
  ga.slot_w = reinterpret_cast<float*>(ws + W.slot_w);
  ga.rnorm = sa.rnorm;
  ga.x = ra.x;
  ga.hbuf = reinterpret_cast<float*>(ws + W.hbuf);
  ga.E = E;
  ga.I = L->I;
  ga.Is = L->Is;
  ga.T = T;
  ga.d = d;
  ga.n_kg = d / 256;
  ga.bits = L->bits;
  ga.hI = W.nbI * 32;
  ga.code_off = ra.code_off;
  ga.has_shared = L->Is > 0;
  ga.am = am;
  {
    // one workgroup per CU (the kernel's LDS allows no more), never more
    // workgroups than 16-row tiles
    const int max_items = (W.max_slots - (ga.has_shared ? 1 : 0)) * (L->I / 16) + (ga.has_shared ? L->Is / 16 : 0);
    int n_wg = env_int("MOE_GU_WGS", cu_count());
    if (n_wg > max_items) n_wg = max_items;
    if (n_wg < 1) n_wg = 1;
    // workgroups set apart for the shared expert's items (one per four of
    // its 16-row tiles: two k-parts per item), which then start without
    // waiting for the selection
    int sh = ga.has_shared ? env_int("MOE_GU_SHARED_WGS", (L->Is / 16 + 3) / 4) : 0;
    if (sh < 0) sh = 0;
    if (sh > L->Is / 16) sh = L->Is / 16;
    if (sh > n_wg / 4) sh = n_wg / 4;
    ga.sh_wgs = sh;
    timed_begin(0, s, &slot);
    serial_point(s);
    HIPCHK(launch_gu_decode(ga, n_wg, s));
  }
  timed_end(slot, s);

  DownArgs da{};
  da.X = X;
  da.n_slots = ga.n_slots;
  da.slot_expert = ga.slot_expert;
  da.hbuf = ga.hbuf;
  da.E = E;
  da.d = d;
  da.T = T;
  da.bits = L->bits;
  da.hI = ga.hI;
  da.BK = L->ex.down.BK;
  da.RT = L->ex.down.RT;
  da.n_kg_r = L->ex.down.n_kg;
  da.n_kg_s = L->Is > 0 ? L->sh.down.n_kg : 0;
  da.S = W.S;
  da.has_shared = L->Is > 0;
  da.max_slots = W.max_slots;
  da.am = am;
  da.ypart = reinterpret_cast<float*>(ws + W.ypart);
  int dn_nw = env_int("MOE_DOWN_WAVES", 8);
  if (dn_nw <= 0 || dn_nw > 8) dn_nw = 8;
  timed_begin(1, s, &slot);
  serial_point(s);
  HIPCHK(launch_down_decode(da, L->ex.down.n_rg, dn_nw, s));
  timed_end(slot, s);
  *S_out = W.S;
  return MOE_OK;
}

// The next layer's routing-independent weights: router rows (fp16 hi and
// lo, the form the prefill router reads) and the shared expert.
static WarmArgs next_layer_lines(const moe_layer* L) {
  WarmArgs a{};
  const int64_t rb = (int64_t)L->E16 * L->d * 2;
  a.p[0] = reinterpret_cast<const uint8_t*>(L->router_wh);
  a.bytes[0] = rb;
  a.p[1] = reinterpret_cast<const uint8_t*>(L->router_wl);
  a.bytes[1] = rb;
  a.p[2] = L->shared;
  a.bytes[2] = L->Is > 0 ? L->sh.bytes : 0;
  a.n = L->Is > 0 ? 3 : 2;
  return a;
}

// One prefill layer (T > 8): prep -> router -> top-k -> group -> gate/up ->
// down -> combine into y.  next: the layer after this one in a stack, whose
// routing-independent weights the gate/up kernel's idle workgroups read
// ahead, or null.
int prefill_layer(const moe_layer* L, const float* x, int norm, float eps, int T, float* y, const moe_route_io* r,
                  uint8_t* ws, hipStream_t s, const moe_layer* next = nullptr) {
  const PfLayout W = ws_layout_prefill(L, T);
  const int d = L->d, E = L->E, k = L->k;
  const bool forced = r && r->in_idx && r->in_w;
  int slot;

  PfPrepArgs pa{};
  pa.x = x;
  pa.T = T;
  pa.d = d;
  pa.norm = norm;
  pa.eps = eps;
  pa.ex = reinterpret_cast<int32_t*>(ws + W.ex);
  pa.xh = reinterpret_cast<_Float16*>(ws + W.xh);
  pa.xl = reinterpret_cast<_Float16*>(ws + W.xl);
  serial_point(s);
  HIPCHK(launch_pf_prep(pa, s));

  const int32_t* idx;
  const float* w;
  if (forced) {
    idx = r->in_idx;
    w = r->in_w;
  } else {
    PfRouterArgs ra{};
    ra.xh = pa.xh;
    ra.xl = pa.xl;
    ra.ex = pa.ex;
    ra.wh = L->router_wh;
    ra.wl = L->router_wl;
    ra.ew = L->router_ew;
    ra.bias = L->router_b;
    ra.T = T;
    ra.d = d;
    ra.E = E;
    ra.E16 = L->E16;
    ra.logits = (r && r->out_logits) ? r->out_logits : reinterpret_cast<float*>(ws + W.logits);
    ra.split = router_split(L, T);
    ra.part = reinterpret_cast<float*>(ws + W.rpart);
    // a split router (short chunks) hands its slice sums straight to the
    // selection kernel, which forms the logits and selects
    const bool fused = pf_router_topk_ok(ra);
    timed_begin(5, s, &slot);
    serial_point(s);
    HIPCHK(launch_pf_router(ra, s, !fused));
    timed_end(slot, s);
    int32_t* oi = (r && r->out_idx) ? r->out_idx : reinterpret_cast<int32_t*>(ws + W.idx);
    float* ow = (r && r->out_w) ? r->out_w : reinterpret_cast<float*>(ws + W.w);
    serial_point(s);
    if (fused) HIPCHK(launch_pf_router_topk(ra, k, oi, ow, s));
    else HIPCHK(launch_topk(ra.logits, T, E, k, oi, ow, s));
    idx = oi;
    w = ow;
  }
  if (forced && r->out_idx) HIPCHK(hipMemcpyAsync(r->out_idx, idx, (size_t)T * k * 4, hipMemcpyDeviceToDevice, s));
  if (forced && r->out_w) HIPCHK(hipMemcpyAsync(r->out_w, w, (size_t)T * k * 4, hipMemcpyDeviceToDevice, s));

  PfGroupArgs ga{};
  ga.idx = idx;
  ga.w = w;
  ga.T = T;
  ga.E = E;
  ga.k = k;
  ga.pad = 16;
  ga.TM = PF_TM;
  ga.has_shared = L->Is > 0;
  ga.n_tiles = W.n_tiles;
  ga.tile_bm = reinterpret_cast<uint64_t*>(ws + W.tile_bm);
  ga.tile_cnt = reinterpret_cast<int32_t*>(ws + W.tile_cnt);
  ga.counts = reinterpret_cast<int32_t*>(ws + W.counts);
  ga.offsets = reinterpret_cast<int32_t*>(ws + W.offsets);
  ga.row_src = reinterpret_cast<int32_t*>(ws + W.row_src);
  ga.row_tok = reinterpret_cast<int32_t*>(ws + W.row_tok);
  ga.row_w = reinterpret_cast<float*>(ws + W.row_w);
  ga.slot_pos = reinterpret_cast<int32_t*>(ws + W.slot_pos);
  ga.n_items = reinterpret_cast<int32_t*>(ws + W.n_items);
  ga.item_group = reinterpret_cast<int32_t*>(ws + W.item_group);
  ga.item_row0 = reinterpret_cast<int32_t*>(ws + W.item_row0);
  ga.item_rows = reinterpret_cast<int32_t*>(ws + W.item_rows);
  ga.R_fill = 0;
  serial_point(s);
  HIPCHK(launch_pf_group(ga, s));

  PfGemmArgs ma{};
  ma.X = expert_set(L);
  ma.xh = pa.xh;
  ma.ex = pa.ex;
  ma.row_tok = ga.row_tok;
  ma.row_w = ga.row_w;
  ma.n_items = ga.n_items;
  ma.item_group = ga.item_group;
  ma.item_row0 = ga.item_row0;
  ma.item_rows = ga.item_rows;
  ma.T = T;
  ma.d = d;
  ma.E = E;
  ma.I = L->I;
  ma.Is = L->Is;
  ma.nbH = W.nbH;
  ma.n_nt = W.n_nt;
  ma.R = W.R;
  ma.hfrag = reinterpret_cast<_Float16*>(ws + W.hfrag);
  ma.hb = L->hbound;
  ma.ed = L->dbound;
  ma.yh = reinterpret_cast<_Float16*>(ws + W.ypart);
  ma.rowf = reinterpret_cast<float*>(ws + W.rowf);
  if (next) ma.warm = next_layer_lines(next);
  timed_begin(3, s, &slot);
  serial_point(s);
  HIPCHK(launch_pf_gate_up(ma, L->bits, W.max_items, s));
  timed_end(slot, s);
  timed_begin(4, s, &slot);
  serial_point(s);
  HIPCHK(launch_pf_down(ma, L->bits, L->ex.down.BK, W.max_items, s));
  timed_end(slot, s);

  PfCombineArgs ca{};
  ca.yh = ma.yh;
  ca.rowf = ma.rowf;
  ca.slot_pos = ga.slot_pos;
  ca.offsets = ga.offsets;
  ca.T = T;
  ca.d = d;
  ca.k = k;
  ca.E = E;
  ca.has_shared = L->Is > 0;
  ca.y = y;
  serial_point(s);
  HIPCHK(launch_pf_combine(ca, s));
  return MOE_OK;
}

// Workspace for calls of up to T tokens through n layers at a time (the
// persistent pass keeps per-layer buffers for up to MOE_PERSIST_MAX_LAYERS).
size_t ws_need(const moe_layer* L, int T, int n_layers) {
  const int Tw = T < 1 ? 1 : T;
  // the decode layouts (8 tokens with fp16 hi + lo activations, 16 with fp16
  // or with fp16 hi + lo activations) and, above 8 tokens, the prefill layout
  const int t8 = Tw < MOE_MAX_TOK_DECODE ? Tw : MOE_MAX_TOK_DECODE, t16 = Tw < MOE_MAX_TOK_F16ACT ? Tw : MOE_MAX_TOK_F16ACT;
  size_t dec = std::max((size_t)ws_layout_decode(L, t8).total, (size_t)ws_layout_decode(L, t16, MOE_AM_F16).total);
  dec = std::max(dec, (size_t)ws_layout_decode(L, t16, MOE_AM_HL16).total);
  dec = std::max(dec, (size_t)std::max(ws_layout_persist(L, t8, false, n_layers).total,
                                       ws_layout_persist(L, t16, true, n_layers).total));
  return T > MOE_MAX_TOK_DECODE ? std::max(dec, (size_t)ws_layout_prefill(L, T).total) : dec;
}

int check_ws(const moe_layer* L, int T, int n_layers, void* ws, size_t ws_bytes, size_t* need) {
  if (T > MOE_MAX_TOK_PREFILL) return fail(MOE_ERR_UNSUPPORTED, "T above %d not supported", MOE_MAX_TOK_PREFILL);
  *need = ws_need(L, T, n_layers);
  if (!ws) return fail(MOE_ERR_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < *need) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, *need);
  return MOE_OK;
}

}  // namespace

// ------------------------------------------------------ allocation-free ---
// Device scratch of moe_layer_forward_noalloc: a file-scope device array that
// every such call on a GPU shares (each GPU holds its own copy until the
// process ends).  Its name is a host-side stand-in in host code, not a device
// address: the address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of this device's scratch (looked up on the first call on
// each device).
int scratch_ptr(void** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_packed_bytes(const moe_layer_desc* desc, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return fail(MOE_ERR_ARG, "bytes is NULL");
  moe_expert_layout ex{}, sh{};
  const int bkd = down_bk(desc->d_ff, desc->d_ff_shared);
  if (!make_expert(desc->d_model, desc->d_ff, desc_kind(desc), &ex, bkd))
    return fail(MOE_ERR_UNSUPPORTED, "expert shape not tileable");
  if (desc->d_ff_shared > 0 && !make_expert(desc->d_model, desc->d_ff_shared, desc_kind(desc), &sh, bkd))
    return fail(MOE_ERR_UNSUPPORTED, "shared expert shape not tileable");
  *bytes = (size_t)packed_layout(desc, ex, sh).total;
  return MOE_OK;
}

static int pack_layer(const moe_layer_desc* desc, const void* experts_canon, const void* shared_canon,
                      const uint8_t* grid, const float* router_w, const float* router_bias, void* packed,
                      size_t packed_bytes, moe_layer** out, void* stream) {
  size_t need = 0;
  int rc = moe_packed_bytes(desc, &need);
  if (rc) return rc;
  if (!out) return fail(MOE_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (desc->codebook && !grid) return fail(MOE_ERR_ARG, "codebook blocks need a grid (moe_pack_experts_cb)");
  if (!experts_canon || !router_w || !packed) return fail(MOE_ERR_ARG, "experts_canon, router_w and packed must be non-NULL");
  if ((desc->d_ff_shared > 0) != (shared_canon != nullptr))
    return fail(MOE_ERR_ARG, "shared_canon must be given exactly when d_ff_shared > 0");
  if (!aligned(packed, 256)) return fail(MOE_ERR_ARG, "packed must be 256-byte aligned");
  if (!aligned(router_w, 16) || (router_bias && !aligned(router_bias, 4)))
    return fail(MOE_ERR_ARG, "router_w must be 16-byte aligned");
  if (packed_bytes < need) return fail(MOE_ERR_ARG, "packed buffer too small: %zu < %zu", packed_bytes, need);
  init_kernels();
  if (g_init_err != hipSuccess) return fail(MOE_ERR_HIP, "kernel init: %s", hipGetErrorString(g_init_err));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  moe_layer* L = new (std::nothrow) moe_layer{};
  if (!L) return fail(MOE_ERR_ARG, "out of host memory");
  L->d = desc->d_model;
  L->E = desc->n_experts;
  L->I = desc->d_ff;
  L->Is = desc->d_ff_shared;
  L->k = desc->top_k;
  L->bits = desc_kind(desc);
  const int bkd = down_bk(L->I, L->Is);
  make_expert(L->d, L->I, L->bits, &L->ex, bkd);
  if (L->Is > 0) make_expert(L->d, L->Is, L->bits, &L->sh, bkd);
  const PackedLayout P = packed_layout(desc, L->ex, L->sh);
  uint8_t* base = reinterpret_cast<uint8_t*>(packed);
  L->packed = base;
  L->packed_bytes = (size_t)P.total;
  L->router_w = reinterpret_cast<const float*>(base + P.off_rw);
  L->router_b = reinterpret_cast<const float*>(base + P.off_rb);
  L->router_wh = reinterpret_cast<const _Float16*>(base + P.off_rwh);
  L->router_wl = reinterpret_cast<const _Float16*>(base + P.off_rwl);
  L->router_ew = reinterpret_cast<const int32_t*>(base + P.off_rew);
  L->hbound = reinterpret_cast<const int32_t*>(base + P.off_hb);
  L->dbound = L->hbound + (L->E + 1);
  L->E16 = e16_of(L->E);
  L->experts = base + P.off_ex;
  L->shared = L->Is > 0 ? base + P.off_sh : nullptr;
  L->grid16 = desc->codebook ? reinterpret_cast<const uint32_t*>(base + P.off_grid) : nullptr;

  auto bail = [&](int code) { delete L; return code; };
  uint32_t* status = reinterpret_cast<uint32_t*>(base + P.off_status);
  hipError_t e;
  if ((e = launch_fill_u32(status, 64, 0u, s)) != hipSuccess) return bail(fail(MOE_ERR_HIP, "fill: %s", hipGetErrorString(e)));
  if ((e = hipMemcpyAsync(base + P.off_rw, router_w, (size_t)L->E * L->d * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "router copy: %s", hipGetErrorString(e)));
  if (router_bias) {
    if ((e = hipMemcpyAsync(base + P.off_rb, router_bias, (size_t)L->E * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return bail(fail(MOE_ERR_HIP, "bias copy: %s", hipGetErrorString(e)));
  } else if ((e = launch_fill_u32(reinterpret_cast<uint32_t*>(base + P.off_rb), (size_t)L->E, 0u, s)) != hipSuccess) {
    return bail(fail(MOE_ERR_HIP, "bias fill: %s", hipGetErrorString(e)));
  }
  if ((e = launch_pack_router(router_w, L->E, L->d, const_cast<_Float16*>(L->router_wh),
                              const_cast<_Float16*>(L->router_wl), const_cast<int32_t*>(L->router_ew), s)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "router split: %s", hipGetErrorString(e)));
  const int64_t bb = canon_block_bytes(L->bits);
  if (L->grid16 &&
      (e = launch_pack_grid(grid, reinterpret_cast<uint16_t*>(const_cast<uint32_t*>(L->grid16)), status, s)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "grid: %s", hipGetErrorString(e)));
  {
    int32_t* hb = const_cast<int32_t*>(L->hbound);
    int32_t* edp = const_cast<int32_t*>(L->dbound);
    const int64_t stride = 3 * (int64_t)L->I * (L->d / 32) * bb;
    if ((e = launch_pack_hbound(reinterpret_cast<const uint8_t*>(experts_canon), stride, L->E, L->I, L->d, L->bits, grid,
                                hb, edp, s)) != hipSuccess)
      return bail(fail(MOE_ERR_HIP, "bound: %s", hipGetErrorString(e)));
    if (L->Is > 0) {
      if ((e = launch_pack_hbound(reinterpret_cast<const uint8_t*>(shared_canon), 0, 1, L->Is, L->d, L->bits, grid,
                                  hb + L->E, edp + L->E, s)) != hipSuccess)
        return bail(fail(MOE_ERR_HIP, "bound: %s", hipGetErrorString(e)));
    } else {
      if ((e = launch_fill_u32(reinterpret_cast<uint32_t*>(hb + L->E), 1, 0u, s)) != hipSuccess ||
          (e = launch_fill_u32(reinterpret_cast<uint32_t*>(edp + L->E), 1, 0u, s)) != hipSuccess)
        return bail(fail(MOE_ERR_HIP, "bound fill: %s", hipGetErrorString(e)));
    }
  }
  auto pack_expert = [&](const uint8_t* canon, int I, const moe_expert_layout& X, uint8_t* dst, int n) -> hipError_t {
    const int64_t gate_b = (int64_t)I * (L->d / 32) * bb;
    const int64_t canon_stride = 3 * gate_b;
    hipError_t r;
    if ((r = launch_pack_matrix(canon, canon_stride, dst + X.off_gate, X.bytes, n, X.gate, L->bits, status, s)) != hipSuccess) return r;
    if ((r = launch_pack_matrix(canon + gate_b, canon_stride, dst + X.off_up, X.bytes, n, X.up, L->bits, status, s)) != hipSuccess) return r;
    return launch_pack_matrix(canon + 2 * gate_b, canon_stride, dst + X.off_down, X.bytes, n, X.down, L->bits, status, s);
  };
  if ((e = pack_expert(reinterpret_cast<const uint8_t*>(experts_canon), L->I, L->ex, base + P.off_ex, L->E)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "pack: %s", hipGetErrorString(e)));
  if (L->Is > 0 && (e = pack_expert(reinterpret_cast<const uint8_t*>(shared_canon), L->Is, L->sh, base + P.off_sh, 1)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "pack shared: %s", hipGetErrorString(e)));
  uint32_t flag = 0;
  if ((e = hipMemcpyAsync(&flag, status, 4, hipMemcpyDeviceToHost, s)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "status copy: %s", hipGetErrorString(e)));
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return bail(fail(MOE_ERR_HIP, "sync: %s", hipGetErrorString(e)));
  if (flag & 1u)
    return bail(fail(MOE_ERR_DATA, "a block scale is inf/nan or has magnitude >= %d", L->bits == MOE_KIND_CB ? 256 : 8192));
  if (flag & 2u) return bail(fail(MOE_ERR_DATA, "a codebook magnitude is above 127"));
  *out = L;
  return MOE_OK;
}

int moe_pack_experts(const moe_layer_desc* desc, const void* experts_canon, const void* shared_canon,
                     const float* router_w, const float* router_bias, void* packed, size_t packed_bytes,
                     moe_layer** out, void* stream) {
  return pack_layer(desc, experts_canon, shared_canon, nullptr, router_w, router_bias, packed, packed_bytes, out,
                    stream);
}

int moe_pack_experts_cb(const moe_layer_desc* desc, const void* experts_canon, const void* shared_canon,
                        const uint8_t* grid, const float* router_w, const float* router_bias, void* packed,
                        size_t packed_bytes, moe_layer** out, void* stream) {
  if (desc && !desc->codebook) return fail(MOE_ERR_ARG, "moe_pack_experts_cb needs desc->codebook = 1");
  if (!grid || !aligned(grid, 16)) return fail(MOE_ERR_ARG, "grid must be non-NULL and 16-byte aligned");
  return pack_layer(desc, experts_canon, shared_canon, grid, router_w, router_bias, packed, packed_bytes, out, stream);
}

int moe_layer_release(moe_layer* layer) {
  delete layer;
  return MOE_OK;
}

int moe_layer_get_desc(const moe_layer* L, moe_layer_desc* out) {
  if (!L || !out) return fail(MOE_ERR_ARG, "NULL argument");
  out->d_model = L->d;
  out->n_experts = L->E;
  out->d_ff = L->I;
  out->d_ff_shared = L->Is;
  out->top_k = L->k;
  out->bits = L->bits == MOE_KIND_CB ? 3 : L->bits;
  out->block = 32;
  out->codebook = L->bits == MOE_KIND_CB;
  return MOE_OK;
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, void* stream) {
  if (T < 0) return fail(MOE_ERR_ARG, "T must be >= 0");
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_ARG, "E must be in [1, %d]", MOE_MAX_E);
  if (k < 1 || k > E || k > MOE_MAX_K) return fail(MOE_ERR_ARG, "k must be in [1, min(E, %d)]", MOE_MAX_K);
  if (T == 0) return MOE_OK;
  if (!logits || !idx || !w) return fail(MOE_ERR_ARG, "NULL pointer");
  if (!aligned(logits, 4) || !aligned(idx, 4) || !aligned(w, 4)) return fail(MOE_ERR_ARG, "misaligned pointer");
  HIPCHK(launch_topk(logits, T, E, k, idx, w, reinterpret_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_workspace_bytes(const moe_layer* L, int T, size_t* bytes) {
  if (!L || !bytes) return fail(MOE_ERR_ARG, "NULL argument");
  if (T < 0) return fail(MOE_ERR_ARG, "T must be >= 0");
  if (T > MOE_MAX_TOK_PREFILL) return fail(MOE_ERR_UNSUPPORTED, "T above %d not supported", MOE_MAX_TOK_PREFILL);
  *bytes = ws_need(L, T, MOE_PERSIST_MAX_LAYERS);
  return MOE_OK;
}

int moe_layer_workspace_bytes(const moe_layer* L, int T, size_t* bytes) {
  if (!L || !bytes) return fail(MOE_ERR_ARG, "NULL argument");
  if (T < 0) return fail(MOE_ERR_ARG, "T must be >= 0");
  if (T > MOE_MAX_TOK_PREFILL) return fail(MOE_ERR_UNSUPPORTED, "T above %d not supported", MOE_MAX_TOK_PREFILL);
  *bytes = ws_need(L, T, 1);
  return MOE_OK;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned(ws, 256)) return fail(MOE_ERR_ARG, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < 256) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  // control words: the first ctrl_bytes() of any workspace
  size_t n = (size_t)ctrl_bytes();
  if (n > ws_bytes) n = ws_bytes;
  HIPCHK(launch_fill_u32(reinterpret_cast<uint32_t*>(ws), n / 4, 0u, reinterpret_cast<hipStream_t>(stream)));
  return MOE_OK;
}

// Argument checks shared by the layer entry points.
static int layer_args(const moe_layer* L, const float* x, int T, float* y, const moe_route_io* route, void* ws,
                      size_t ws_bytes) {
  if (!L) return fail(MOE_ERR_ARG, "layer is NULL");
  if (T < 0) return fail(MOE_ERR_ARG, "T must be >= 0");
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_ERR_ARG, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(MOE_ERR_ARG, "x and y must be 16-byte aligned");
  const char* xb = reinterpret_cast<const char*>(x);
  const char* yb = reinterpret_cast<const char*>(y);
  const size_t nbytes = (size_t)T * L->d * 4;
  if (xb < yb + nbytes && yb < xb + nbytes) return fail(MOE_ERR_ARG, "x and y must not alias");
  if (route && ((route->in_idx == nullptr) != (route->in_w == nullptr)))
    return fail(MOE_ERR_ARG, "in_idx and in_w must be given together");
  size_t need;
  int rc = check_ws(L, T, 1, ws, ws_bytes, &need);
  if (rc) return rc;
  init_kernels();
  if (g_init_err != hipSuccess) return fail(MOE_ERR_HIP, "kernel init: %s", hipGetErrorString(g_init_err));
  return MOE_OK;
}

// One decode pass of T tokens and the combine of the down splits into y.
// The persistent pass applies to layers of one shape with at most 1024
// experts; it runs where MOE_PERSIST=1 is set in the environment (the
// per-phase kernels are the default: they measure faster on the 48-layer,
// 8-token stack).
static bool persist_usable(const moe_layer* const* layers, int n_layers) {
  if (env_int("MOE_PERSIST", 0) == 0 || persist_grid() <= 0) return false;
  const moe_layer* L = layers[0];
  if (!persist_supported(L->E, L->bits)) return false;
  for (int l = 1; l < n_layers; ++l) {
    const moe_layer* M = layers[l];
    if (M->d != L->d || M->E != L->E || M->I != L->I || M->Is != L->Is || M->k != L->k || M->bits != L->bits)
      return false;
  }
  return true;
}

// One decode pass of T tokens through layers[0..n) by the persistent kernel,
// in launches of up to MOE_PERSIST_MAX_LAYERS layers (a later launch takes the
// previous one's split partials as its input).  x, y point at the pass's first
// row; layer l's output goes to y_layers + l * yl_stride, its routing to
// idx_layers / w_layers + l * route_stride.  r: one-layer routing input and
// outputs (n_layers == 1), or null.
static int persist_pass(const moe_layer* const* layers, int n_layers, const float* x, int T, float eps, float* y,
                        float* y_layers, int64_t yl_stride, int32_t* idx_layers, float* w_layers, int64_t route_stride,
                        const moe_route_io* r, uint8_t* ws, hipStream_t s, bool act16) {
  const moe_layer* L = layers[0];
  const PsLayout W = ws_layout_persist(L, T, act16, n_layers);
  const int R = act16 ? MOE_MAX_TOK_F16ACT : MOE_MAX_TOK_DECODE;
  const int d = L->d;
  PersistArgs P{};
  P.off_wh = reinterpret_cast<const uint8_t*>(L->router_wh) - L->packed;
  P.off_wl = reinterpret_cast<const uint8_t*>(L->router_wl) - L->packed;
  P.off_ew = reinterpret_cast<const uint8_t*>(L->router_ew) - L->packed;
  P.off_br = reinterpret_cast<const uint8_t*>(L->router_b) - L->packed;
  P.off_ex = L->experts - L->packed;
  P.off_sh = L->Is > 0 ? L->shared - L->packed : 0;
  P.ex_stride = L->ex.bytes;
  P.off_gate = L->ex.off_gate;
  P.off_up = L->ex.off_up;
  P.off_down = L->ex.off_down;
  P.sh_off_gate = L->sh.off_gate;
  P.sh_off_up = L->sh.off_up;
  P.sh_off_down = L->sh.off_down;
  P.T = T;
  P.d = d;
  P.E = L->E;
  P.k = L->k;
  P.I = L->I;
  P.Is = L->Is;
  P.bits = L->bits;
  P.has_shared = L->Is > 0;
  P.code_off = moe_code_offset(L->bits);
  P.n_cs = W.n_cs;
  P.n_rs = W.n_rs;
  P.S = W.S;
  P.n_rg = L->ex.down.n_rg;
  P.n_kg_r = L->ex.down.n_kg;
  P.n_kg_s = L->Is > 0 ? L->sh.down.n_kg : 0;
  P.max_slots = W.max_slots;
  P.hI = W.hI;
  P.cpl = W.cpl;
  P.eps = eps;
  P.yl_stride = yl_stride;
  P.route_stride = route_stride;
  const bool forced = r && r->in_idx && r->in_w;
  P.out_logits = (r && !forced) ? r->out_logits : nullptr;
  P.in_idx = forced ? r->in_idx : nullptr;
  P.in_w = forced ? r->in_w : nullptr;
  P.lp = reinterpret_cast<float*>(ws + W.lp);
  P.ss_part = reinterpret_cast<float*>(ws + W.ss_part);
  P.rnorm = reinterpret_cast<float*>(ws + W.rnorm);
  P.logits = reinterpret_cast<float*>(ws + W.logits);
  P.x.frag = reinterpret_cast<_Float16*>(ws + W.xfrag);
  P.x.cs = reinterpret_cast<float*>(ws + W.xcs);
  P.x.sx = reinterpret_cast<int32_t*>(ws + W.xsx);
  P.hbuf = reinterpret_cast<float*>(ws + W.hbuf);
  P.logits_stride = W.logits_stride;
  P.logits_row = logits_row(L->E);
  P.xfrag_stride = W.xfrag_stride;
  P.xcs_stride = W.xcs_stride;
  P.xsx_stride = W.xsx_stride;
  P.hbuf_stride = W.hbuf_stride;
  P.ctl = reinterpret_cast<uint32_t*>(ws + W.ctl);
  P.ypart = reinterpret_cast<float*>(ws + W.ypart);
  P.status = reinterpret_cast<uint32_t*>(ws + W.ctrl + kStatusOffset);
  const size_t clear_words = W.clear_words;
  for (int l0 = 0; l0 < n_layers; l0 += MOE_PERSIST_MAX_LAYERS) {
    const int nl = n_layers - l0 < MOE_PERSIST_MAX_LAYERS ? n_layers - l0 : MOE_PERSIST_MAX_LAYERS;
    P.n_layers = nl;
    for (int i = 0; i < nl; ++i) P.base[i] = layers[l0 + i]->packed;
    P.in = l0 == 0 ? x : P.ypart;
    P.S_in = l0 == 0 ? 1 : W.S;
    P.in_stride = l0 == 0 ? 0 : (int64_t)R * d;
    P.norm0 = l0 > 0;
    P.y = l0 + nl == n_layers ? y : nullptr;
    P.y_prev_out = (l0 > 0 && y_layers) ? y_layers + (size_t)(l0 - 1) * yl_stride : nullptr;
    P.y_layers = y_layers ? y_layers + (size_t)l0 * yl_stride : nullptr;
    P.idx_layers = idx_layers ? idx_layers + (size_t)l0 * route_stride : nullptr;
    P.w_layers = w_layers ? w_layers + (size_t)l0 * route_stride : nullptr;
    int slot;
    timed_begin(6, s, &slot);
    serial_point(s);
    HIPCHK(launch_persist(P, L->ex.down.RT, persist_grid(), act16, clear_words, s));
    timed_end(slot, s);
  }
  return MOE_OK;
}

// Tokens 9..16 of a full-precision call take one decode pass with 16 hi + lo
// token rows (MOE_MID_T=0 in the environment: the grouped GEMMs for a layer,
// passes of 8 tokens for a stack, as before the 16-row pass existed).
static bool mid_t_decode() { return env_int("MOE_MID_T", 1) != 0; }

static int decode_layer_out(const moe_layer* L, const float* x, int T, float* y, const moe_route_io* route,
                            uint8_t* wsb, hipStream_t st, int am) {
  if (am != MOE_AM_HL16 && persist_usable(&L, 1)) {
    int32_t* oi = route ? route->out_idx : nullptr;
    float* ow = route ? route->out_w : nullptr;
    return persist_pass(&L, 1, x, T, 0.f, y, nullptr, 0, oi, ow, 0, route, wsb, st, am == MOE_AM_F16);
  }
  int S = 1;
  int rc = decode_layer(L, LayerInput{x, 1, 0, 0}, 0.f, T, nullptr, route, wsb, st, &S, am);
  if (rc) return rc;
  const WsLayout W = ws_layout_decode(L, T, am);
  const int64_t R = moe_am_tokens(am);
  HIPCHK(launch_combine(reinterpret_cast<const float*>(wsb + W.ypart), S, R * L->d, T, L->d, y, st));
  return MOE_OK;
}

int moe_layer_forward(const moe_layer* L, const float* x, int T, float* y, const moe_route_io* route, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = layer_args(L, x, T, y, route, ws, ws_bytes);
  if (rc || T == 0) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  if (T > MOE_MAX_TOK_DECODE && T <= MOE_MAX_TOK_F16ACT && mid_t_decode())
    return decode_layer_out(L, x, T, y, route, wsb, st, MOE_AM_HL16);
  if (T > MOE_MAX_TOK_DECODE) return prefill_layer(L, x, 0, 0.f, T, y, route, wsb, st);
  return decode_layer_out(L, x, T, y, route, wsb, st, MOE_AM_HL8);
}

int moe_layer_forward_noalloc(const moe_layer* L, const float* x, int T, float* y, const moe_route_io* route,
                              void* stream) {
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc) return rc;
  rc = layer_args(L, x, T, y, route, ws, MOE_NOALLOC_SCRATCH_BYTES);
  if (rc || T == 0) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  // the scratch keeps the previous call's contents: clear the control words
  // the kernels count in (a fill kernel, so the call stays capturable)
  HIPCHK(launch_fill_u32(reinterpret_cast<uint32_t*>(wsb), (size_t)ctrl_bytes() / 4, 0u, st));
  if (T > MOE_MAX_TOK_DECODE && T <= MOE_MAX_TOK_F16ACT && mid_t_decode())
    return decode_layer_out(L, x, T, y, route, wsb, st, MOE_AM_HL16);
  if (T > MOE_MAX_TOK_DECODE) return prefill_layer(L, x, 0, 0.f, T, y, route, wsb, st);
  return decode_layer_out(L, x, T, y, route, wsb, st, MOE_AM_HL8);
}

int moe_layer_forward_f16act(const moe_layer* L, const float* x, int T, float* y, const moe_route_io* route,
                             void* ws, size_t ws_bytes, void* stream) {
  if (T > MOE_MAX_TOK_F16ACT) return fail(MOE_ERR_UNSUPPORTED, "T above %d not supported with fp16 activations", MOE_MAX_TOK_F16ACT);
  int rc = layer_args(L, x, T, y, route, ws, ws_bytes);
  if (rc || T == 0) return rc;
  return decode_layer_out(L, x, T, y, route, reinterpret_cast<uint8_t*>(ws), reinterpret_cast<hipStream_t>(stream),
                          MOE_AM_F16);
}

// Argument checks shared by the stack entry points.
static int stack_args(const moe_layer* const* layers, int n_layers, const float* x, int T, float* y,
                      float* y_layers, int32_t* idx_layers, float* w_layers, void* ws, size_t ws_bytes) {
  if (!layers || n_layers < 1) return fail(MOE_ERR_ARG, "need at least one layer");
  if (T < 0) return fail(MOE_ERR_ARG, "T must be >= 0");
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_ERR_ARG, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || (y_layers && !aligned(y_layers, 16)))
    return fail(MOE_ERR_ARG, "x, y and y_layers must be 16-byte aligned");
  if ((idx_layers == nullptr) != (w_layers == nullptr)) return fail(MOE_ERR_ARG, "idx_layers and w_layers go together");
  const int d = layers[0] ? layers[0]->d : 0;
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l]) return fail(MOE_ERR_ARG, "layer %d is NULL", l);
    if (layers[l]->d != d) return fail(MOE_ERR_ARG, "layer %d has d_model %d, expected %d", l, layers[l]->d, d);
    size_t need;
    int rc = check_ws(layers[l], T, n_layers, ws, ws_bytes, &need);
    if (rc) return rc;
  }
  init_kernels();
  if (g_init_err != hipSuccess) return fail(MOE_ERR_HIP, "kernel init: %s", hipGetErrorString(g_init_err));
  return MOE_OK;
}

// The decode kernels, the whole stack for up to `chunk` tokens at a time
// (rows are independent); chunk rows sit at row c0 of x, y, y_layers[l] and
// the routing outputs.
static int decode_stack(const moe_layer* const* layers, int n_layers, const float* x, int T, float eps, float* y,
                        float* y_layers, int32_t* idx_layers, float* w_layers, uint8_t* wsb, hipStream_t s,
                        int am) {
  const int d = layers[0]->d;
  const int chunk = moe_am_tokens(am);
  const bool act16 = am == MOE_AM_F16;
  if (am != MOE_AM_HL16 && persist_usable(layers, n_layers)) {
    const int k = layers[0]->k;
    for (int c0 = 0; c0 < T; c0 += chunk) {
      const int Tc = T - c0 < chunk ? T - c0 : chunk;
      int rc = persist_pass(layers, n_layers, x + (size_t)c0 * d, Tc, eps, y + (size_t)c0 * d,
                            y_layers ? y_layers + (size_t)c0 * d : nullptr, (int64_t)T * d,
                            idx_layers ? idx_layers + (size_t)c0 * k : nullptr,
                            w_layers ? w_layers + (size_t)c0 * k : nullptr, (int64_t)T * k, nullptr, wsb, s, act16);
      if (rc) return rc;
    }
    return MOE_OK;
  }
  for (int c0 = 0; c0 < T; c0 += chunk) {
    const int Tc = T - c0 < chunk ? T - c0 : chunk;
    LayerInput in{x + (size_t)c0 * d, 1, 0, 0};
    for (int l = 0; l < n_layers; ++l) {
      moe_route_io r{};
      if (idx_layers) {
        r.out_idx = idx_layers + ((size_t)l * T + c0) * layers[l]->k;
        r.out_w = w_layers + ((size_t)l * T + c0) * layers[l]->k;
      }
      float* prev_out = (l > 0 && y_layers) ? y_layers + ((size_t)(l - 1) * T + c0) * d : nullptr;
      int S = 1;
      int rc = decode_layer(layers[l], in, eps, Tc, prev_out, &r, wsb, s, &S, am);
      if (rc) return rc;
      const WsLayout W = ws_layout_decode(layers[l], Tc, am);
      in = LayerInput{reinterpret_cast<const float*>(wsb + W.ypart), S, (int64_t)chunk * d, 1};
    }
    serial_point(s);
    HIPCHK(launch_combine(in.p, in.S, in.stride, Tc, d, y + (size_t)c0 * d, s));
    if (y_layers)
      HIPCHK(hipMemcpyAsync(y_layers + ((size_t)(n_layers - 1) * T + c0) * d, y + (size_t)c0 * d, (size_t)Tc * d * 4,
                            hipMemcpyDeviceToDevice, s));
  }
  return MOE_OK;
}

int moe_stack_forward(const moe_layer* const* layers, int n_layers, const float* x, int T, float eps, float* y,
                      float* y_layers, int32_t* idx_layers, float* w_layers, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = stack_args(layers, n_layers, x, T, y, y_layers, idx_layers, w_layers, ws, ws_bytes);
  if (rc || T == 0) return rc;
  const int d = layers[0]->d;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  if (T > MOE_MAX_TOK_CHUNKED) {
    // Layer l reads h_l (x, then the previous output) and writes y_layers[l]
    // or y; the RMSNorm of the input is fused into the layer's prep step.
    // Reading and writing y in one layer is safe: the prep step consumes its
    // input before the combine step writes the output.
    // While layer l computes, its gate/up kernel's workgroups without a work
    // item read layer l + 1's router rows and shared expert into the
    // Infinity Cache (MOE_PREFETCH=0 in the environment turns this off).
    const bool ahead = env_int("MOE_PREFETCH", 1) != 0;
    for (int l = 0; l < n_layers; ++l) {
      moe_route_io r{};
      if (idx_layers) {
        r.out_idx = idx_layers + (size_t)l * T * layers[l]->k;
        r.out_w = w_layers + (size_t)l * T * layers[l]->k;
      }
      const float* in = l == 0 ? x : (y_layers ? y_layers + (size_t)(l - 1) * T * d : y);
      float* out = y_layers ? y_layers + (size_t)l * T * d : y;
      rc = prefill_layer(layers[l], in, l > 0, eps, T, out, &r, wsb, s,
                         ahead && l + 1 < n_layers ? layers[l + 1] : nullptr);
      if (rc) return rc;
    }
    if (y_layers) HIPCHK(hipMemcpyAsync(y, y_layers + (size_t)(n_layers - 1) * T * d, (size_t)T * d * 4, hipMemcpyDeviceToDevice, s));
    return MOE_OK;
  }
  const int am = T > MOE_MAX_TOK_DECODE && mid_t_decode() ? MOE_AM_HL16 : MOE_AM_HL8;
  return decode_stack(layers, n_layers, x, T, eps, y, y_layers, idx_layers, w_layers, wsb, s, am);
}

int moe_stack_forward_f16act(const moe_layer* const* layers, int n_layers, const float* x, int T, float eps,
                             float* y, float* y_layers, int32_t* idx_layers, float* w_layers, void* ws,
                             size_t ws_bytes, void* stream) {
  if (T > MOE_MAX_TOK_F16ACT) return fail(MOE_ERR_UNSUPPORTED, "T above %d not supported with fp16 activations", MOE_MAX_TOK_F16ACT);
  int rc = stack_args(layers, n_layers, x, T, y, y_layers, idx_layers, w_layers, ws, ws_bytes);
  if (rc || T == 0) return rc;
  return decode_stack(layers, n_layers, x, T, eps, y, y_layers, idx_layers, w_layers, reinterpret_cast<uint8_t*>(ws),
                      reinterpret_cast<hipStream_t>(stream), MOE_AM_F16);
}

int moe_group_workspace_bytes(int T, int E, int k, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_ARG, "bytes is NULL");
  if (T < 0 || T > MOE_MAX_TOK_PREFILL) return fail(MOE_ERR_ARG, "T must be in [0, %d]", MOE_MAX_TOK_PREFILL);
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_ARG, "E must be in [1, %d]", MOE_MAX_E);
  if (k < 1 || k > MOE_MAX_K) return fail(MOE_ERR_ARG, "k must be in [1, %d]", MOE_MAX_K);
  const int64_t n_tiles = (T + PF_T64 - 1) / PF_T64;
  *bytes = (size_t)(moe_align256(n_tiles * E * 8) + moe_align256(n_tiles * E * 4));
  if (*bytes == 0) *bytes = 256;
  return MOE_OK;
}

int moe_group_tokens(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                     void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  int rc = moe_group_workspace_bytes(T, E, k, &need);
  if (rc) return rc;
  if (!counts || !offsets) return fail(MOE_ERR_ARG, "counts and offsets must be non-NULL");
  if (T > 0 && (!idx || !perm)) return fail(MOE_ERR_ARG, "idx and perm must be non-NULL");
  if (!ws || !aligned(ws, 256)) return fail(MOE_ERR_ARG, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
  if (!aligned(idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4))
    return fail(MOE_ERR_ARG, "misaligned pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int n_tiles = (T + PF_T64 - 1) / PF_T64;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  PfGroupArgs ga{};
  ga.idx = idx;
  ga.T = T;
  ga.E = E;
  ga.k = k;
  ga.pad = 1;
  ga.TM = PF_TM;
  ga.n_tiles = n_tiles;
  ga.tile_bm = reinterpret_cast<uint64_t*>(wsb);
  ga.tile_cnt = reinterpret_cast<int32_t*>(wsb + moe_align256((int64_t)n_tiles * E * 8));
  ga.counts = counts;
  ga.offsets = offsets;
  ga.row_src = perm;
  ga.R_fill = T * k;
  if (T == 0) {
    HIPCHK(launch_fill_u32(reinterpret_cast<uint32_t*>(counts), (size_t)E, 0u, s));
    HIPCHK(launch_fill_u32(reinterpret_cast<uint32_t*>(offsets), (size_t)E + 1, 0u, s));
    return MOE_OK;
  }
  HIPCHK(launch_pf_group(ga, s));
  return MOE_OK;
}

int moe_rmsnorm(const float* x, int T, int d, float eps, float* y, void* stream) {
  if (T < 0 || d <= 0 || d % 4) return fail(MOE_ERR_ARG, "need T >= 0 and d a positive multiple of 4");
  if (T == 0) return MOE_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return fail(MOE_ERR_ARG, "x, y must be non-NULL and 16-byte aligned");
  HIPCHK(launch_rmsnorm(x, T, d, eps, y, reinterpret_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_debug_unpack(const moe_layer* L, int expert, int mat, int8_t* codes, float* w_f32, uint16_t* w_f16,
                     void* stream) {
  if (!L) return fail(MOE_ERR_ARG, "layer is NULL");
  if (expert < -1 || expert >= L->E) return fail(MOE_ERR_ARG, "expert out of range");
  if (expert == -1 && L->Is == 0) return fail(MOE_ERR_ARG, "layer has no shared expert");
  if (mat < 0 || mat > 2) return fail(MOE_ERR_ARG, "mat must be 0, 1 or 2");
  if (!codes && !w_f32 && !w_f16) return MOE_OK;
  const moe_expert_layout& X = expert < 0 ? L->sh : L->ex;
  const uint8_t* base = expert < 0 ? L->shared : L->experts + (int64_t)expert * L->ex.bytes;
  const moe_mat_layout& M = mat == 0 ? X.gate : mat == 1 ? X.up : X.down;
  const int64_t off = mat == 0 ? X.off_gate : mat == 1 ? X.off_up : X.off_down;
  HIPCHK(launch_debug_unpack(base + off, reinterpret_cast<const uint16_t*>(L->grid16), M, L->bits, codes, w_f32, w_f16,
                             reinterpret_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_debug_unpack_path(const moe_layer* L, int expert, int mat, int path, int8_t* codes, float* w_f32,
                          uint16_t* w_f16, void* stream) {
  if (!L) return fail(MOE_ERR_ARG, "layer is NULL");
  if (expert < -1 || expert >= L->E) return fail(MOE_ERR_ARG, "expert out of range");
  if (expert == -1 && L->Is == 0) return fail(MOE_ERR_ARG, "layer has no shared expert");
  if (mat < 0 || mat > 2) return fail(MOE_ERR_ARG, "mat must be 0, 1 or 2");
  if (path < 0 || path > 2) return fail(MOE_ERR_ARG, "path must be 0, 1 or 2");
  if (path == 0 && w_f16) return fail(MOE_ERR_ARG, "path 0 exports codes and w_f32 only");
  if (path > 0 && (codes || w_f32)) return fail(MOE_ERR_ARG, "paths 1 and 2 export w_f16 only");
  if (!codes && !w_f32 && !w_f16) return MOE_OK;
  const moe_expert_layout& X = expert < 0 ? L->sh : L->ex;
  const uint8_t* base = expert < 0 ? L->shared : L->experts + (int64_t)expert * L->ex.bytes;
  const moe_mat_layout& M = mat == 0 ? X.gate : mat == 1 ? X.up : X.down;
  const int64_t off = mat == 0 ? X.off_gate : mat == 1 ? X.off_up : X.off_down;
  DebugPathArgs a{};
  a.mat = base + off;
  a.grid16 = L->grid16;
  a.cols = M.cols;
  a.BK = M.BK;
  a.RT = M.RT;
  a.n_rg = M.n_rg;
  a.n_kg = M.n_kg;
  a.chunk_bytes = M.chunk_bytes;
  a.full = path == 2;
  a.codes = codes;
  a.w32 = w_f32;
  a.w16 = w_f16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (path == 0) HIPCHK(launch_debug_decode_path(a, L->bits, s));
  else HIPCHK(launch_debug_prefill_path(a, L->bits, s));
  return MOE_OK;
}

int moe_workspace_status(const void* ws, size_t ws_bytes, int* status, void* stream) {
  if (!ws || !status || !aligned(ws, 256)) return fail(MOE_ERR_ARG, "workspace and status must be non-NULL (workspace 256-byte aligned)");
  if (ws_bytes < (size_t)ctrl_bytes()) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t v = 0;
  HIPCHK(hipMemcpyAsync(&v, reinterpret_cast<const uint8_t*>(ws) + kStatusOffset, 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  *status = v ? 1 : 0;
  return MOE_OK;
}

int moe_timing_start(int kernel_class, int max_launches) {
  if (kernel_class < 0 || kernel_class > 6 || max_launches < 1) return fail(MOE_ERR_ARG, "bad timing arguments");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (hipEvent_t e : g_timing.ev) hipEventDestroy(e);
  g_timing.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : g_timing.ev) HIPCHK(hipEventCreate(&e));
  g_timing.max = max_launches;
  g_timing.used = 0;
  g_timing.cls = kernel_class;
  return MOE_OK;
}

int moe_timing_stop(double* total_ms, int* launches) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  const int cls = g_timing.cls;
  g_timing.cls = -1;
  if (cls < 0) return fail(MOE_ERR_ARG, "timing not started");
  double tot = 0;
  for (int i = 0; i < g_timing.used; ++i) {
    HIPCHK(hipEventSynchronize(g_timing.ev[2 * i + 1]));
    float ms = 0;
    HIPCHK(hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]));
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = g_timing.used;
  for (hipEvent_t e : g_timing.ev) hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.used = 0;
  return MOE_OK;
}

}  // extern "C"
