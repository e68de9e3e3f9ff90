// moe_launch.h -- kernel argument blocks and host-side launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

// Largest number of expert slots a decode call can touch: up to 8 tokens x 16
// routed experts, plus the shared expert.
#define MOE_MAX_SLOTS (MOE_MAX_TOK_DECODE * MOE_MAX_K + 1)
// Columns of the layer input handled by one route workgroup.
#define MOE_ROUTE_COLS 256
// Expert rows per route workgroup (4 waves x 16 rows).
#define MOE_ROUTE_ROWS 64
// Most down-projection splits (partial sums a consumer adds up).
#define MOE_MAX_IN_SPLITS 16
// Most column slices of the router (d <= 8192).
#define MOE_MAX_CS 32

// ---------------------------------------------------------------- decode ---
// Layer input: in = sum over S_in splits of in[s * in_stride + t * d + j]
// (the previous layer's down partials, or the caller's x with S_in = 1).
struct RouteArgs {
  const float* in;
  int32_t S_in;
  int64_t in_stride;  // floats between splits
  const float* Wr;    // [E][d]
  int32_t T, d, E, code_off, do_logits;
  float* lp;        // ws [d/256][T][E] partial logits
  float* ss_part;   // ws [d/256][T] partial sums of squares
  _Float16* xfrag;  // ws [d/32][64][8]
  float* xsum;      // ws [d/32][16]
  float* y_out;     // optional: the summed input, [T][d]
};

struct SelectArgs {
  const float* lp;       // [n_cs][T][E]
  const float* ss_part;  // [n_cs][T]
  const float* br;       // [E]
  int32_t n_cs, T, d, E, k, norm;
  float eps;
  const int32_t* fidx;  // forced routing or null
  const float* fw;
  float* logits;  // ws [T][E]
  int32_t* idx;   // ws [T][k]
  float* w;       // ws [T][k]
  float* rnorm;   // ws [8]: per-token divisor (1 when norm == 0)
  float* out_logits;
  int32_t* out_idx;
  float* out_w;
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
  const int32_t* idx;  // [T][k]
  const float* w;      // [T][k]
  int32_t k;
  int32_t* n_slots;      // out [1]
  int32_t* slot_expert;  // out [MAX_SLOTS]
  float* slot_w;         // out [MAX_SLOTS][8]
  const float* rnorm;
  const _Float16* xfrag;
  const float* xsum;
  _Float16* hfrag;  // ws [MAX_SLOTS][nbI][64][8]
  float* hsum;      // ws [MAX_SLOTS][nbI][16]
  int32_t E, I, Is, T, n_kg, bits, nbI, code_off, has_shared;
};

struct DownArgs {
  ExpertSet X;
  const int32_t* n_slots;
  const int32_t* slot_expert;
  const _Float16* hfrag;
  const float* hsum;
  int32_t E, d, T, bits, nbI, BK, RT, n_kg_r, n_kg_s, S, has_shared;
  float* ypart;  // ws [S][8][d]
};

hipError_t launch_pack_matrix(const uint8_t* canon, int64_t canon_stride, uint8_t* out, int64_t out_stride,
                              int n_experts, const moe_mat_layout& L, int bits, uint32_t* bad_scale,
                              hipStream_t s);
hipError_t launch_debug_unpack(const uint8_t* mat, const moe_mat_layout& L, int bits, int8_t* codes, float* w32,
                               uint16_t* w16, hipStream_t s);

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_gu_decode(const GuArgs& a, int n_wg, hipStream_t s);
hipError_t launch_down_decode(const DownArgs& a, int grid_x, int nw, hipStream_t s);
hipError_t launch_combine(const float* part, int S, int64_t stride, int T, int d, float* y, hipStream_t s);

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int T, int d, float eps, float* y, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
hipError_t moe_route_kernels_init();
