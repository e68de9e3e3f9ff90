// moe_launch.h -- kernel argument blocks and host-side launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

// Largest number of expert slots a decode call can touch: up to 8 tokens x 16
// routed experts, plus the shared expert.
#define MOE_MAX_SLOTS (MOE_MAX_TOK_DECODE * MOE_MAX_K + 1)

// ---------------------------------------------------------------- decode ---
struct RouteArgs {
  const float* x;  // layer input [T][d]
  int32_t norm;    // 1: the input is the previous layer's output, normalise first
  float eps;
  const float* Wr;  // [E][d]
  const float* br;  // [E]
  int32_t T, d, E, k, has_shared, code_off, rows_per_wg;
  const int32_t* fidx;  // forced routing or null
  const float* fw;
  float* logits;  // ws [T][E]
  int32_t* idx;   // ws [T][k]
  float* w;       // ws [T][k]
  float* out_logits;
  int32_t* out_idx;
  float* out_w;
  int32_t* n_slots;      // ws [1]
  int32_t* slot_expert;  // ws [MAX_SLOTS]
  float* slot_w;         // ws [MAX_SLOTS][8]
  _Float16* xfrag;       // ws [d/32][64][8]
  float* xsum;           // ws [d/32][16]
  uint32_t* counter;     // ws, zero between calls
};

struct ExpertSet {
  const uint8_t* experts;  // routed expert 0
  int64_t ex_stride;       // bytes per routed expert
  const uint8_t* shared;   // shared expert or null
  int64_t off_gate, off_up, off_down;           // routed
  int64_t sh_off_gate, sh_off_up, sh_off_down;  // shared
};

struct GuArgs {
  ExpertSet X;
  const int32_t* n_slots;
  const int32_t* slot_expert;
  const float* slot_w;
  const _Float16* xfrag;
  const float* xsum;
  _Float16* hfrag;  // ws [MAX_SLOTS][nbI][64][8]
  float* hsum;      // ws [MAX_SLOTS][nbI][16]
  int32_t E, I, Is, n_kg, bits, nbI, code_off;
};

struct DownArgs {
  ExpertSet X;
  const int32_t* n_slots;
  const int32_t* slot_expert;
  const _Float16* hfrag;
  const float* hsum;
  int32_t E, d, T, bits, nbI, BK, RT, n_kg_r, n_kg_s, S;
  float* y;          // [T][d]
  float* ypart;      // ws [S][8][d]
  uint32_t* counters;  // ws [d / (16 RT)], zero between calls
};

hipError_t launch_pack_matrix(const uint8_t* canon, int64_t canon_stride, uint8_t* out, int64_t out_stride,
                              int n_experts, const moe_mat_layout& L, int bits, uint32_t* bad_scale,
                              hipStream_t s);
hipError_t launch_debug_unpack(const uint8_t* mat, const moe_mat_layout& L, int bits, int8_t* codes, float* w32,
                               uint16_t* w16, hipStream_t s);

hipError_t launch_route_decode(const RouteArgs& a, int n_wg, hipStream_t s);
hipError_t launch_gu_decode(const GuArgs& a, int grid_x, int grid_y, int nw, hipStream_t s);
hipError_t launch_down_decode(const DownArgs& a, int grid_x, int nw, hipStream_t s);

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int T, int d, float eps, float* y, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
hipError_t moe_route_kernels_init();
