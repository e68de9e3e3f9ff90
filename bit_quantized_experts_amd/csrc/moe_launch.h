// moe_launch.h -- kernel argument blocks and host-side launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "moe_internal.h"

// Largest number of expert slots a decode pass can touch: up to 16 tokens
// (fp16 activations) x 16 routed experts, plus the shared expert.
#define MOE_MAX_SLOTS (MOE_MAX_TOK_F16ACT * MOE_MAX_K + 1)
// Columns of the layer input handled by one route workgroup.
#define MOE_ROUTE_COLS 128
// Expert rows per route workgroup (4 waves x 16 rows).
#define MOE_ROUTE_ROWS 64
// Most down-projection splits (partial sums a consumer adds up).
#define MOE_MAX_IN_SPLITS 8
// Most column slices of the router (d <= 8192).
#define MOE_MAX_CS 64
// Control words of the workspace used by the route kernel: one completion
// counter per row slice (E <= 4096: at most 64).
#define MOE_CTRL_WORDS 64

// ---------------------------------------------------------------- decode ---
// Layer input: in = sum over S_in splits of in[s * in_stride + t * d + j]
// (the previous layer's down partials, or the caller's x with S_in = 1).
struct SelectArgs {
  float* ss_part;      // [n_rs][n_cs][T] sums of squares, one copy per row slice
  const float* br;     // [E]
  const int32_t* ew;   // [E16] router row exponents (partial logits are unscaled)
  int32_t n_cs, n_rs, T, d, E, norm;
  float eps;
  uint32_t* ctrl;      // completion counters, one per row slice; zero between calls
  float* logits;       // ws [T][E]
  float* rnorm;        // ws [16]: per-token divisor (1 when norm == 0)
  float* out_logits;   // optional copy of the logits
};

struct RouteArgs {
  const float* in;
  int32_t S_in;
  int64_t in_stride;  // floats between splits
  const _Float16* wh;  // router rows times 2^-ew, fp16 hi part, B-fragments [E16/16][d/32][64][8]
  const _Float16* wl;  // same, lo part
  int32_t T, d, E, code_off, do_logits;
  int32_t act16;    // 1: gate/up A-fragments hold 16 tokens in fp16 (else 8 tokens as fp16 hi + lo)
  float* lp;        // ws [d/MOE_ROUTE_COLS][T][E] partial logits
  _Float16* xfrag;  // ws [d/32][64][8]
  float* xsum;      // ws [d/32][16]
  float* y_out;     // optional: the summed input, [T][d]
  SelectArgs sel;   // the logits, finished by the last workgroup of each row slice
};

struct ExpertSet {
  const uint8_t* experts;  // routed expert 0
  int64_t ex_stride;       // bytes per routed expert
  const uint8_t* shared;   // shared expert or null
  int64_t off_gate, off_up, off_down;           // routed
  int64_t sh_off_gate, sh_off_up, sh_off_down;  // shared
};

// Slot list of a decode layer: slot 0 is the shared expert (if any), then the
// distinct routed experts in ascending id order; slot_w[u][t] is token t's
// gate weight for slot u (0 = not routed there).  Built by every gate/up
// workgroup from the routing; workgroup 0 publishes it for the down kernel.
struct GuArgs {
  ExpertSet X;
  const float* logits;  // [T][E]: every workgroup selects the top k itself; or null:
  const int32_t* idx;   // [T][k] forced routing (ids out of range are skipped)
  const float* w;       // [T][k]
  int32_t* out_idx;     // optional: the selection ([T][k], written by workgroup 0)
  float* out_w;
  int32_t k;
  int32_t* n_slots;      // out [1]
  int32_t* slot_expert;  // out [MAX_SLOTS]
  float* slot_w;         // out [MAX_SLOTS][16]
  const float* rnorm;
  const _Float16* xfrag;
  const float* xsum;
  _Float16* hfrag;  // ws [MAX_SLOTS][nbI][64][8]
  float* hsum;      // ws [MAX_SLOTS][2 nbI][16], one row of sums per 16-row tile
  int32_t E, I, Is, T, n_kg, bits, nbI, code_off, has_shared;
  int32_t act16;  // 1: A rows are 16 tokens in fp16 (else 8 tokens as fp16 hi + lo)
};

struct DownArgs {
  ExpertSet X;
  const int32_t* n_slots;
  const int32_t* slot_expert;
  const _Float16* hfrag;
  const float* hsum;
  int32_t E, d, T, bits, nbI, BK, RT, n_kg_r, n_kg_s, S, has_shared, max_slots;
  int32_t act16;  // 1: A rows are 16 tokens in fp16 (else 8 tokens as fp16 hi + lo)
  float* ypart;   // ws [S][R][d], R = 16 with act16, else 8
};

hipError_t launch_pack_matrix(const uint8_t* canon, int64_t canon_stride, uint8_t* out, int64_t out_stride,
                              int n_experts, const moe_mat_layout& L, int bits, uint32_t* bad_scale,
                              hipStream_t s);
hipError_t launch_debug_unpack(const uint8_t* mat, const moe_mat_layout& L, int bits, int8_t* codes, float* w32,
                               uint16_t* w16, hipStream_t s);

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_gu_decode(const GuArgs& a, int n_wg, hipStream_t s);
hipError_t launch_down_decode(const DownArgs& a, int grid_x, int nw, hipStream_t s);
hipError_t launch_combine(const float* part, int S, int64_t stride, int T, int d, float* y, hipStream_t s);

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int T, int d, float eps, float* y, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
hipError_t moe_route_kernels_init();

// --------------------------------------------------------------- prefill ---
// Chunked prefill (T > 8): the routed (token, slot) pairs are grouped by
// expert into rows; each expert's rows are padded to a multiple of 16 and cut
// into work items of up to PF_TM rows; the shared expert's rows (one per
// token, in token order) follow the routed rows.
#define PF_TM 128   // rows per work item
#define PF_HT 128   // intermediate columns per gate/up workgroup (4 waves x 32)
#define PF_DT 256   // output columns per down workgroup (4 waves x 64)
#define PF_ET 128   // experts per router workgroup (4 waves x 32)
#define PF_T64 64   // tokens per grouping tile

struct PfPrepArgs {
  const float* x;  // [T][d]
  int32_t T, d, norm;
  float eps;
  int32_t* ex;     // [T] power-of-two exponent of the row
  _Float16* xh;    // [T][d] fp16(x * 2^-ex)
  _Float16* xl;    // [T][d] fp16(x * 2^-ex - xh)
};

struct PfRouterArgs {
  const _Float16* xh;
  const _Float16* xl;
  const int32_t* ex;
  const _Float16* wh;  // router hi/lo fragments [E16/16][d/32][64][8]
  const _Float16* wl;
  const int32_t* ew;   // [E16] row exponents
  const float* bias;   // [E]
  int32_t T, d, E, E16;
  float* logits;  // [T][E]
  // split = 1: one workgroup per 256-column slice (blockIdx.z) writes that
  // slice's unscaled sums to part [d/256][T][E]; a reduce kernel adds them
  int32_t split;
  float* part;
};

struct PfGroupArgs {
  const int32_t* idx;  // [T][k]
  const float* w;      // [T][k] or null
  int32_t T, E, k, pad, TM, has_shared, n_tiles;
  uint64_t* tile_bm;   // [n_tiles][E] token bitmaps of each expert
  int32_t* tile_cnt;   // [n_tiles][E] counts, then exclusive prefix over tiles
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E + 2]: padded row offsets; [E] routed rows, [E+1] all rows
  int32_t* row_src;    // [R] t*k + r of the row, -1 for padding / shared rows
  int32_t* row_tok;    // [R] token of the row (0 for padding), or null
  float* row_w;        // [R] gate weight of the row (shared 1, padding 0), or null
  int32_t* slot_pos;   // [T*k] row of each pair, -1 if not used, or null
  int32_t* n_items;    // [1] or null (no work list)
  int32_t* item_group; // [max_items] expert (E = shared)
  int32_t* item_row0;
  int32_t* item_rows;  // multiple of 16, <= TM
  int32_t R_fill;      // rows of row_src to fill with -1 beyond the routed rows (export)
};

struct PfGemmArgs {
  ExpertSet X;
  const _Float16* xh;     // gate/up: activation rows
  const int32_t* ex;      // gate/up: row exponents of x
  const int32_t* row_tok;
  const float* row_w;
  const int32_t* n_items;
  const int32_t* item_group;
  const int32_t* item_row0;
  const int32_t* item_rows;
  const int32_t* hb;  // [E + 1] per-expert exponent base of the intermediate rows (index E: shared)
  const int32_t* ed;  // [E + 1] per-expert exponent of the down rows (index E: shared)
  int32_t T, d, E, I, Is, nbH, n_nt, R;
  _Float16* hfrag;   // [R/16][nbH][64][8] intermediate rows, fp16(h * 2^-(hb + 2 ex))
  _Float16* yh;      // [R][d] down rows, fp16(sum * 2^-ed)
  float* rowf;       // [R] factor of each down row: w * 2^(hb + 2 ex + ed)
};

struct PfCombineArgs {
  const _Float16* yh;
  const float* rowf;
  const int32_t* slot_pos;
  const int32_t* offsets;  // offsets[E] = first shared row
  int32_t T, d, k, E, has_shared;
  float* y;
};

hipError_t launch_pack_router(const float* W, int E, int d, _Float16* wh, _Float16* wl, int32_t* ew, hipStream_t s);
hipError_t launch_pack_hbound(const uint8_t* canon, int64_t canon_stride, int n_experts, int I, int d, int bits,
                              int32_t* hb, int32_t* ed, hipStream_t s);
hipError_t launch_pf_prep(const PfPrepArgs& a, hipStream_t s);
hipError_t launch_pf_router(const PfRouterArgs& a, hipStream_t s);
hipError_t launch_pf_group(const PfGroupArgs& a, hipStream_t s);
hipError_t launch_pf_gate_up(const PfGemmArgs& a, int bits, int max_items, hipStream_t s);
hipError_t launch_pf_down(const PfGemmArgs& a, int bits, int bk, int max_items, hipStream_t s);
hipError_t launch_pf_combine(const PfCombineArgs& a, hipStream_t s);

// Events that the next launch of the kernel class being timed records itself
// (start and end of its dispatch, as a profiler sees them); null otherwise.
// Set by the host code around one launch, never during graph capture.
struct MoeLaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local MoeLaunchEvents moe_launch_events;

#define MOE_LAUNCH(K, grid, block, shmem, s, ...)                                                        \
  do {                                                                                                   \
    if (moe_launch_events.start)                                                                         \
      hipExtLaunchKernelGGL(K, grid, block, shmem, s, moe_launch_events.start, moe_launch_events.stop, 0, \
                            __VA_ARGS__);                                                                \
    else                                                                                                 \
      hipLaunchKernelGGL(K, grid, block, shmem, s, __VA_ARGS__);                                         \
  } while (0)
