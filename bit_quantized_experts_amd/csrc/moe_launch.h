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
// Activation rows of the decode kernels' matrix-core A operand (the `am`
// argument fields): 8 tokens as fp16 hi + lo rows (one 16-row tile per
// 32-input block), 16 tokens rounded to fp16 (one tile), or 16 tokens as fp16
// hi + lo rows (two tiles per block: tokens 0..7 and 8..15, each weight
// fragment multiplied by both).
#define MOE_AM_HL8 0
#define MOE_AM_F16 1
#define MOE_AM_HL16 2
constexpr int moe_am_tokens(int am) { return am == MOE_AM_HL8 ? 8 : 16; }
constexpr int moe_am_tiles(int am) { return am == MOE_AM_HL16 ? 2 : 1; }

// The layer input as the gate/up kernel's matrix-core A operand, written by
// the router's row-slice-0 workgroups (one per column slice of
// MOE_ROUTE_COLS inputs): every 32-input block as NT tiles of [64 lanes][8]
// fp16 (NT = moe_am_tiles(am); in tile tt lane m + 16q holds inputs
// 8q..8q+7 of row m: the fp16 hi part of token 8tt + m for m < 8 and the lo
// part of token 8tt + m - 8 for m >= 8, or token m rounded to fp16 with fp16
// rows), the tiles' accumulator seeds (-2^(b-1) times the row sums of the
// block), and the power of two 2^-e every (column slice, token) was scaled
// by before the split (e from the slice's largest magnitude of the token:
// 2^14 <= max 2^-e < 2^15).
#define MOE_XSX_STRIDE 64  // words between two slices' exponents (a 256-byte line each)
struct XFrag {
  _Float16* frag;  // [d/32][NT][64][8]
  float* cs;       // [d/32][NT][16]
  int32_t* sx;     // [d/MOE_ROUTE_COLS][MOE_XSX_STRIDE], token t at t
};

// Layer input: in = sum over S_in splits of in[s * in_stride + t * d + j]
// (the previous layer's down partials, or the caller's x with S_in = 1).
struct SelectArgs {
  float* ss_part;      // [n_rs][n_cs][T] sums of squares, one copy per row slice
  const float* br;     // [E]
  const int32_t* ew;   // [E16] router row exponents (partial logits are unscaled)
  int32_t n_cs, n_rs, T, d, E, norm;
  float eps;
  uint32_t* ctrl;      // completion counters, one per row slice; zero between calls
  int32_t ctrl_stride; // words between two of them
  float* logits;       // ws [T][logits_stride]
  int32_t logits_stride;  // floats per token row: E rounded up to a multiple of 64 (a row
                          // slice's 64 logits fill whole lines of their own)
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
  int32_t am;       // activation rows of the gate/up A operand (MOE_AM_*)
  float* lp;        // ws [d/MOE_ROUTE_COLS][T][E] partial logits
  XFrag x;          // the gate/up kernel's A operand (row slice 0 writes it)
  float* y_out;     // optional: the summed input, [T][d]
  SelectArgs sel;   // the logits, finished by the last workgroup of each row slice
};

struct ExpertSet {
  const uint8_t* experts;  // routed expert 0
  int64_t ex_stride;       // bytes per routed expert
  const uint8_t* shared;   // shared expert or null
  int64_t off_gate, off_up, off_down;           // routed
  int64_t sh_off_gate, sh_off_up, sh_off_down;  // shared
  const uint32_t* grid16;  // codebook blocks: [512][2] words, 4 fp16 magnitudes per entry (else null)
};

// Slot list of a decode layer: slot 0 is the shared expert (if any), then the
// distinct routed experts in ascending id order; slot_w[u][t] is token t's
// gate weight for slot u (0 = not routed there).  Built by every gate/up
// workgroup from the routing; workgroup 0 publishes it for the down kernel.
struct GuArgs {
  ExpertSet X;
  const float* logits;  // [T][logits_stride]: every workgroup selects the top k itself; or null:
  int32_t logits_stride;
  const int32_t* idx;   // [T][k] forced routing (ids out of range are skipped)
  const float* w;       // [T][k]
  int32_t* out_idx;     // optional: the selection ([T][k], written by workgroup 0)
  float* out_w;
  int32_t k;
  int32_t* n_slots;      // out [1]
  int32_t* slot_expert;  // out [MAX_SLOTS]
  float* slot_w;         // out [MAX_SLOTS][16]
  const float* rnorm;
  XFrag x;               // the layer input as A-fragments (before the RMSNorm of stacked layers)
  float* hbuf;      // ws [MAX_SLOTS][hI/16][R][16] fp32 h = w silu(g) u, R = moe_am_tokens(am)
  int32_t E, I, Is, T, d, n_kg, bits, hI, code_off, has_shared;
  int32_t am;  // activation rows (MOE_AM_*)
  int32_t sh_wgs;  // workgroups that run only the shared expert's items (0: none)
};

struct DownArgs {
  ExpertSet X;
  const int32_t* n_slots;
  const int32_t* slot_expert;
  const float* hbuf;       // [MAX_SLOTS][R][hI] fp32
  int32_t E, d, T, bits, hI, BK, RT, n_kg_r, n_kg_s, S, has_shared, max_slots;
  int32_t am;     // activation rows (MOE_AM_*)
  float* ypart;   // ws [S][R][d], R = moe_am_tokens(am)
};

// Block kinds as the kernels' template tag: 2 and 3 are b-bit code blocks,
// MOE_KIND_CB codebook blocks (32 weights: fp16 scale, eight 9-bit indices
// into a grid of 512 entries of 4 magnitudes, 32 sign bits).  A packed chunk
// holds 8 fragments of 16 rows x 32 inputs (4096 weights) in every kind:
// 1280, 1792 and 1920 bytes.
#define MOE_KIND_CB 4
constexpr int moe_chunk_bytes(int kind) { return kind == 2 ? 1280 : kind == 3 ? 1792 : 1920; }
// The unsigned-code offset the accumulator seed removes (0: signed codes).
constexpr int moe_code_offset(int kind) { return kind == MOE_KIND_CB ? 0 : 1 << (kind - 1); }

// Persistent decode pass over up to MOE_PERSIST_MAX_LAYERS layers of one
// shape (persist.hip).  Every layer's packed buffer has the same layout, so a
// layer is its base pointer plus these offsets.
#define MOE_PERSIST_MAX_LAYERS 16
// Words between two counters of the persistent pass (each its own 128-byte
// line, so workgroups polling one counter do not slow the others).
#define MOE_CTR_STRIDE 32
// Words between two layers' per-token words (divisors, exponents): each
// layer's copy has 256-byte lines of its own.  L2-cached reads of a line
// another layer writes later would otherwise return the earlier contents.
#define MOE_PERSIST_TOK_STRIDE 64
struct PersistArgs {
  const uint8_t* base[MOE_PERSIST_MAX_LAYERS];
  int64_t off_wh, off_wl, off_ew, off_br, off_ex, off_sh;
  int64_t ex_stride, off_gate, off_up, off_down, sh_off_gate, sh_off_up, sh_off_down;
  int32_t n_layers, T, d, E, k, I, Is, bits, has_shared, code_off;
  int32_t n_cs, n_rs, S, n_rg, n_kg_r, n_kg_s, max_slots, hI, cpl;
  float eps;
  // input of the first layer: S_in splits at in_stride floats; norm0: the
  // first layer's input is RMS-normalised (it is a previous layer's output)
  const float* in;
  int32_t S_in, norm0;
  int64_t in_stride;
  float* y;           // [T][d] output, or null: the last layer's partials stay in ypart
  float* y_prev_out;  // optional: where the first layer's (summed) input is copied
  float* y_layers;    // optional: layer l's output at y_layers + l * yl_stride
  int64_t yl_stride;
  int32_t* idx_layers;  // optional routing outputs at + l * route_stride
  float* w_layers;
  int64_t route_stride;
  float* out_logits;        // optional logits of the first layer
  const int32_t* in_idx;    // forced routing of a one-layer pass, or null
  const float* in_w;
  // workspace
  float* lp;
  float* ss_part;
  // per layer (a layer's copy is written once per pass, by one workgroup
  // per cache line, and no line holds two layers' words, so its readers may
  // use L2-cached loads): layer l's buffer at base + l * stride
  float* rnorm;      // [n][MOE_PERSIST_TOK_STRIDE]
  float* logits;     // [n][T][logits_row]
  XFrag x;           // layer 0's; layer l's at + l * the strides below
  float* hbuf;       // [n][max_slots][hI/16][R][16]
  int64_t logits_stride, hbuf_stride, xfrag_stride, xcs_stride, xsx_stride;
  int32_t logits_row;  // floats per token row of the logits
  uint32_t* ctl;     // [n_layers][cpl], counters MOE_CTR_STRIDE words apart
  float* ypart;      // [S][R][d]
  uint32_t* status;  // abort word: non-zero once a wait gave up
};
bool persist_supported(int E, int bits);
int persist_blocks_per_cu();
hipError_t launch_persist(const PersistArgs& a, int rt, int grid, bool act16, size_t clear_words, hipStream_t s);

hipError_t launch_pack_matrix(const uint8_t* canon, int64_t canon_stride, uint8_t* out, int64_t out_stride,
                              int n_experts, const moe_mat_layout& L, int bits, uint32_t* bad_scale,
                              hipStream_t s);
hipError_t launch_debug_unpack(const uint8_t* mat, const uint16_t* grid16, const moe_mat_layout& L, int bits,
                               int8_t* codes, float* w32, uint16_t* w16, hipStream_t s);
hipError_t launch_pack_grid(const uint8_t* grid, uint16_t* out, uint32_t* bad, hipStream_t s);



// Test export of one packed matrix through an expert kernel's own decoder.
struct DebugPathArgs {
  const uint8_t* mat;  // packed matrix
  const uint32_t* grid16;  // codebook blocks: the layer's fp16 grid (else null)
  int32_t cols, BK, RT, n_rg, n_kg, chunk_bytes;
  int32_t full;        // prefill: 1 = whole chunks (load_full), 0 = half chunks (load_half)
  int8_t* codes;       // decode: signed codes [rows][cols], or null
  float* w32;          // decode: scale * code [rows][cols], or null
  uint16_t* w16;       // prefill: fp16 bits of the dequantized weight [rows][cols]
};
hipError_t launch_debug_decode_path(const DebugPathArgs& a, int bits, hipStream_t s);
hipError_t launch_debug_prefill_path(const DebugPathArgs& a, int bits, hipStream_t s);

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

// Byte ranges (128-byte aligned starts; a tail below 128 bytes is skipped)
// whose cache lines are loaded once, results discarded (warm_lines).
struct WarmArgs {
  const uint8_t* p[4];
  int64_t bytes[4];
  int32_t n;
};

struct PfGemmArgs {
  ExpertSet X;
  WarmArgs warm;          // gate/up: lines its workgroups without a work item read ahead (n = 0: none)
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
                              const uint8_t* grid, int32_t* hb, int32_t* ed, hipStream_t s);
hipError_t launch_pf_prep(const PfPrepArgs& a, hipStream_t s);
// reduce = false leaves a split launch's slice sums in part for
// launch_pf_router_topk (route.hip), which adds them, writes the logits and
// selects; it takes split launches with E <= 512 and d <= 4096
// (pf_router_topk_ok).
hipError_t launch_pf_router(const PfRouterArgs& a, hipStream_t s, bool reduce = true);
bool pf_router_topk_ok(const PfRouterArgs& a);
hipError_t launch_pf_router_topk(const PfRouterArgs& a, int k, int32_t* idx, float* w, hipStream_t s);
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
