// moe_internal.h -- shared between the host side (moe_api.cpp) and the
// kernels.  Describes the packed device layout of a layer and the workspace
// carve-up.
//
// Packed matrix layout ("tiled").  A matrix of R rows and C = 32*nb input
// columns is cut into row groups of 16*RT rows and k-groups of BK blocks,
// RT*BK = 8.  For each (row group, k-group) one chunk holds, for the 64 lanes
// of a wavefront, everything one lane needs for 8 MFMA fragments of 16 rows x
// 32 inputs: lane l = n + 16*q (n = row within a 16-row tile, q = quarter of
// the 32-input block) owns codes 8q..8q+7 of row n for each fragment
// f = t*BK + j (row tile t, block j of the k-group).
//   bytes [0, 1024)      codes, 16 B per lane (b=2) or the low 2 bits (b=3):
//                        dword p of lane l holds fragments 2p (even) and
//                        2p+1 (odd); code e of the even fragment is at bits
//                        [4e, 4e+2), of the odd fragment at bits [4e+2, 4e+4).
//   bytes [1024, 1280)   scales, fp16 [16 rows n][8 fragments f].
//   bytes [1280, 1792)   (b=3 only) high code bits, 8 B per lane: dword h of
//                        lane l holds fragments 4h..4h+3; code e of fragment
//                        4h+g is at bit 4e+g.
// A 2-bit chunk is 1280 B and a 3-bit chunk 1792 B, exactly the canonical
// size of the same 512 weights*... (8 fragments x 8 codes x 64 lanes).
// Chunks are stored row group major: chunk(rg, kg) at (rg * n_kg + kg).
#pragma once
#include <stddef.h>
#include <stdint.h>

#define MOE_BLOCK 32
// Tokens per decode pass with one 16-row tile of fp16 hi and lo rows.
#define MOE_MAX_TOK_DECODE 8
// Tokens per decode pass with 16 token rows: fp16 activations (one row per
// token), or a tile of hi parts followed by a tile of lo parts.
#define MOE_MAX_TOK_F16ACT 16
// Layers and stacks of up to this many tokens run the decode kernels (faster
// than the grouped GEMMs at these sizes).
#define MOE_MAX_TOK_CHUNKED 16
#define MOE_MAX_TOK_PREFILL 65536
#define MOE_MAX_K 16
#define MOE_MAX_E 4096

struct moe_mat_layout {
  int32_t rows, cols;   // R, C
  int32_t nb;           // C / 32
  int32_t BK, RT;       // blocks per chunk, row tiles per chunk
  int32_t n_rg, n_kg;   // R / (16 RT), nb / BK
  int32_t chunk_bytes;  // 1280 (2-bit) or 1792 (3-bit)
  int64_t bytes;        // n_rg * n_kg * chunk_bytes
};

struct moe_expert_layout {
  moe_mat_layout gate, up, down;
  int64_t off_gate, off_up, off_down;  // within one expert
  int64_t bytes;                       // one expert, padded to 256
};

// Host-side handle (opaque to callers).
struct moe_layer {
  int32_t d, E, I, Is, k;
  int32_t bits;             // block kind: 2, 3 (b-bit codes) or MOE_KIND_CB (codebook blocks)
  const uint32_t* grid16;   // codebook blocks: device [512][4] fp16 magnitudes (else null)
  moe_expert_layout ex;   // routed experts
  moe_expert_layout sh;   // shared expert (valid if Is > 0)
  const uint8_t* packed;  // device base
  const float* router_w;  // device [E][d]
  const float* router_b;  // device [E]
  const _Float16* router_wh;  // device: router rows times 2^-ew, fp16 hi part, MFMA B fragments
  const _Float16* router_wl;  // same, lo part
  const int32_t* router_ew;   // device [E16] row exponents
  const int32_t* hbound;      // device [E + 1] exponent base of the intermediate rows (E: shared)
  const int32_t* dbound;      // device [E + 1] exponent of the prefill down rows (E: shared)
  int32_t E16;                // E rounded up to a multiple of 16
  const uint8_t* experts; // device, E * ex.bytes
  const uint8_t* shared;  // device, sh.bytes or null
  size_t packed_bytes;
};

// Device view of one expert matrix for kernels.
struct moe_dev_mat {
  const uint8_t* base;  // first chunk
  int32_t n_rg, n_kg, BK, RT, chunk_bytes;
};

static inline int64_t moe_align256(int64_t x) { return (x + 255) & ~(int64_t)255; }
