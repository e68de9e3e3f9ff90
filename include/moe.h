/*
 * moe.h -- C ABI of libmoe.so: a sparse mixture-of-experts layer computed
 * directly from low-bit block-quantised expert weights on an MI355X (gfx950).
 *
 * What the layer computes.  Each token x[t] (fp32, length d) is sent to the
 * k experts with the largest router logits out of E small SwiGLU experts, as
 * in the 48-layer, 512-experts-per-layer model that routes about ten experts
 * per token [cnyes profile of Strata, section "Strata 到底是什麼？"], plus
 * one always-on shared expert kept next to the router [same page, section
 * "三層記憶體", part 1].  Expert weights stay in their low-bit blocks and the
 * kernels multiply from them without first expanding them to full precision
 * [strata-mlx wiki, opening feature list, first item; devlabs blog "32GB Mac
 * mini 6 跑 125B 大模型", section 核心技术特点].  Decode and draft
 * verification pass up to eight tokens at once (one real token plus seven
 * drafts) [devlabs blog, section 核心技术特点, MTP item]; prompts are read in
 * chunks of up to 8192 tokens [agentlenshq article, section "Strata 如何让
 * 125 B 模型适配 12-24 GB 显存", last item].
 *
 *   logits[t][e] = x[t] . Wr[e] + bias[e]
 *   idx[t][0..k)  = the k largest logits, ties to the lower expert index
 *   w[t][r]       = softmax of the k selected logits (rank order)
 *   FFN_e(x)      = Wd_e ( silu(Wg_e x) * (Wu_e x) ),  silu(z) = z / (1 + e^-z)
 *   y[t]          = sum_r w[t][r] FFN_{idx[t][r]}(x[t]) + FFN_shared(x[t])
 *
 * Canonical block format (input of moe_pack_experts).  A block holds 32
 * consecutive weights of one matrix row: bytes [0,2) are an IEEE fp16 scale
 * (little endian), bytes [2, 2+4b) are 32 codes of b bits (b = 2 or 3); code j
 * is bits [b*j, b*j+b) of the little-endian bitstream of those bytes and
 * stands for the integer q_j - 2^(b-1).  Weight = scale * (q_j - 2^(b-1)).
 * One expert is gate [I][d], up [I][d], down [d][I] in that order, row-major,
 * each row a run of blocks along the matrix's input dimension.  E experts are
 * stored back to back; the shared expert is a separate buffer of the same
 * layout with its own intermediate size.
 *
 * Codebook blocks (desc.codebook = 1, packed by moe_pack_experts_cb).  The
 * codebook block types that the model files also use multiply magnitudes
 * looked up in a table that ships with the file [strata-mlx wiki, opening
 * feature list, first item ("nine block types"), and credits list (codebook
 * tables)]; this library takes the table as an input.  A block holds 32
 * weights in 15 bytes: [0,2) fp16 scale; [2,10) the low 8 bits of eight 9-bit
 * grid indices, index i covering weights 4i..4i+3; byte 10, bit i = bit 8 of
 * index i; [11,15) 32 sign bits, bit j of the little-endian word set = weight
 * j negative.  Weight j = scale * (+-1) * grid[index][j % 4], grid = 512
 * entries of 4 unsigned magnitudes (bytes, at most 127).  Same expert layout
 * as above with 15-byte blocks.
 *
 * Conventions for every entry point:
 *   - Return value: MOE_OK (0) or a positive MOE_ERR_* code.  On error,
 *     moe_last_error() returns a message for the calling thread.  Nothing is
 *     launched when an argument check fails.  No call aborts the process.
 *   - Device pointers are caller-owned HIP device memory, 16-byte aligned
 *     (checked).  The library never allocates or frees device memory (its one
 *     static device array, the scratch of moe_layer_forward_noalloc, is part
 *     of its code object).
 *   - `stream` is a hipStream_t (NULL = the default stream).  All GPU work is
 *     enqueued asynchronously on it; apart from moe_pack_experts no call waits
 *     for the GPU, and the forward calls may be captured into a HIP graph.
 *   - Host handles (moe_layer) are immutable after packing and may be shared
 *     between threads and streams.  A workspace must not be used by two calls
 *     that can overlap on the GPU.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,          /* bad pointer, size, shape or alignment */
    MOE_ERR_UNSUPPORTED = 2,  /* valid but not supported shape (see moe_packed_bytes) */
    MOE_ERR_WORKSPACE = 3,    /* workspace smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = 4,          /* a HIP runtime call failed */
    MOE_ERR_DATA = 5          /* input data out of contract (e.g. an fp16 scale that is inf/nan) */
};

typedef struct moe_layer_desc {
    int32_t d_model;      /* d: hidden size; multiple of 256 */
    int32_t n_experts;    /* E: routed experts, 1..4096 */
    int32_t d_ff;         /* I: routed-expert intermediate size; multiple of 32 */
    int32_t d_ff_shared;  /* shared-expert intermediate size, multiple of 32, or 0 = none */
    int32_t top_k;        /* k: 1..min(E, 16) */
    int32_t bits;         /* code width b: 2 or 3 (3 with codebook blocks) */
    int32_t block;        /* weights per block: must be 32 */
    int32_t codebook;     /* 0: b-bit code blocks; 1: codebook blocks (see above) */
} moe_layer_desc;

/* Opaque host handle of one packed layer: shapes plus device pointers into
 * the caller's packed buffer. */
typedef struct moe_layer moe_layer;

/* Optional routing inputs/outputs of moe_layer_forward.
 *   in_idx/in_w   [T][k]: if both non-NULL the router is skipped and this
 *                 routing is used (rank order; expert ids should be in
 *                 [0,E) and distinct within a row; an entry outside [0,E)
 *                 is skipped, i.e. contributes nothing, and a repeated id
 *                 uses its first entry only).
 *   out_logits    [T][E]: router logits (ignored when routing is forced).
 *   out_idx/out_w [T][k]: the routing used.
 * Any pointer may be NULL. */
typedef struct moe_route_io {
    const int32_t *in_idx;
    const float *in_w;
    float *out_logits;
    int32_t *out_idx;
    float *out_w;
} moe_route_io;

/* Message describing the last error on this thread ("" if none). */
const char *moe_last_error(void);

/* Bytes of device memory moe_pack_experts needs for one layer.
 * Rejects (MOE_ERR_ARG / MOE_ERR_UNSUPPORTED) d % 256 != 0, d_ff % 32 != 0,
 * d_ff_shared % 32 != 0, k < 1, k > E, k > 16, E > 4096, bits not in {2,3},
 * block != 32, codebook not in {0,1}, codebook with bits != 3. */
int moe_packed_bytes(const moe_layer_desc *desc, size_t *bytes);

/* Re-tile one layer's canonical blocks into the device layout the kernels
 * stream (lossless integer shuffling: codes stay b-bit, scales stay fp16; no
 * weight is expanded to full precision) and copy the router.  Experts stay
 * in the file's own blocks and the kernels multiply from them [strata-mlx
 * wiki, opening feature list, first item].
 *   experts_canon  device, E * expert_bytes canonical bytes
 *   shared_canon   device, canonical bytes of the shared expert, or NULL when
 *                  d_ff_shared == 0
 *   router_w       device fp32 [E][d]
 *   router_bias    device fp32 [E], or NULL for a zero bias
 *   packed         device, packed_bytes >= moe_packed_bytes(); must stay
 *                  alive and unchanged while the handle is used
 *   out            receives a new host handle (release with moe_layer_release)
 * This call synchronises `stream` once at the end: it checks that every scale
 * is a finite fp16 value with |scale| < 8192 (so that scale * code stays in
 * fp16 range) and returns MOE_ERR_DATA otherwise. */
int moe_pack_experts(const moe_layer_desc *desc, const void *experts_canon, const void *shared_canon,
                     const float *router_w, const float *router_bias, void *packed, size_t packed_bytes,
                     moe_layer **out, void *stream);

/* moe_pack_experts for codebook blocks (desc->codebook = 1): the same
 * arguments plus `grid`, device uint8 [512][4] (16-byte aligned), the table
 * of magnitudes the blocks index [strata-mlx wiki, credits list: the
 * codebook tables come with the model files].  The grid is copied into the
 * packed buffer (as exact fp16 values); a magnitude above 127, or a block
 * scale of magnitude 256 or more (so that scale * code stays below 2^15 in
 * fp16, as for b-bit codes), gives MOE_ERR_DATA.  Every forward entry point
 * takes codebook layers (decode and chunked prefill). */
int moe_pack_experts_cb(const moe_layer_desc *desc, const void *experts_canon, const void *shared_canon,
                        const uint8_t *grid, const float *router_w, const float *router_bias, void *packed,
                        size_t packed_bytes, moe_layer **out, void *stream);

/* Free the host handle (the packed device buffer stays the caller's). */
int moe_layer_release(moe_layer *layer);

/* Copy the layer's shape description. */
int moe_layer_get_desc(const moe_layer *layer, moe_layer_desc *out);

/* Top-k selection and gate weights on given logits (the routing step alone;
 * a router that sends each token to about ten of 512 experts [cnyes profile
 * of Strata, section "Strata 到底是什麼？"]):
 *   logits device fp32 [T][E], idx device int32 [T][k], w device fp32 [T][k].
 * Order: logit descending, ties to the lower expert index (-0.0 == +0.0).
 * Gate weights: m = largest selected logit, e_r = exp(l_r - m) computed in
 * fp64 by a fixed argument reduction (by ln 2) and a degree-13 Taylor
 * polynomial, S = sum of e_r in rank order, w_r = fp32(e_r / S).  Bit-exact
 * with a CPU implementation following the same steps.  Logits must be
 * finite (non-finite values give unspecified but in-range indices).
 * 1 <= k <= min(E, 16), 1 <= E <= 4096, T >= 0. */
int moe_route_topk(const float *logits, int T, int E, int k, int32_t *idx, float *w, void *stream);

/* Device scratch needed by moe_layer_forward / moe_stack_forward for up to T
 * tokens per call with this layer's shapes (any number of stacked layers). */
int moe_workspace_bytes(const moe_layer *layer, int T, size_t *bytes);

/* The (smaller) device scratch a one-layer call (moe_layer_forward and its
 * variants) of up to T tokens needs; at most moe_workspace_bytes. */
int moe_layer_workspace_bytes(const moe_layer *layer, int T, size_t *bytes);

/* Clear the control words of a new workspace (enqueued on `stream`).  Must be
 * called once before a workspace is first used, and again if its memory has
 * been used for anything else in between.  The decode kernels count
 * finished workgroups in these words (the first 256 bytes); a workspace whose
 * words are not zero gives wrong logits and routing.  The forward calls
 * leave the control words cleared for the next call. */
int moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* One layer: y[T][d] = MoE(x[T][d]) [cnyes profile of Strata, sections
 * "Strata 到底是什麼？" (routed experts) and "三層記憶體" part 1 (shared
 * expert); devlabs blog, section 核心技术特点, MTP item (eight tokens per
 * verify pass); agentlenshq article, section "Strata 如何让 125 B 模型适配
 * 12-24 GB 显存", last item (8192-token prompt chunks)].  T = 0 is a no-op.
 * T <= 16 runs the
 * decode/verify kernels (experts streamed once per call with 128-bit loads
 * and multiplied from their codes, activations carried as fp16 hi + lo: up
 * to 8 tokens as hi and lo rows of one matrix-core tile, 9..16 tokens as a
 * tile of their hi parts whose products the tile of their lo parts
 * continues, so each weight fragment is decoded once for all 16);
 * 16 < T <= 65536 runs the chunked-prefill kernels: the (token, slot) pairs are grouped by expert (as
 * moe_group_tokens) and each expert's rows go through a grouped matrix
 * multiply on the matrix cores with the weights dequantized in registers to
 * fp16 and the activations rounded to fp16 after an exact per-row
 * power-of-two scaling (fp32 accumulation).  With given routing (in_idx,
 * in_w) a token's row with a repeated expert id uses the first occurrence
 * only, and ids outside [0, E) are skipped.  x and y must not alias.
 * `route` may be NULL.  ws_bytes >= moe_workspace_bytes(layer, T). */
int moe_layer_forward(const moe_layer *layer, const float *x, int T, float *y, const moe_route_io *route,
                      void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * moe_layer_forward with the library's own device scratch instead of a
 * caller's workspace.  The scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends; this call allocates nothing and frees nothing.  Arguments,
 * routing input/output and results as moe_layer_forward (the same kernels).
 * A call whose workspace (moe_layer_workspace_bytes) exceeds the scratch returns
 * MOE_ERR_WORKSPACE before launching anything (a full-size layer of 2560 x
 * 512 experts fits up to 8 tokens; long prefill chunks do not).  Every call
 * on one GPU shares that GPU's scratch: calls that can overlap on one GPU
 * (different streams, or several host threads) race and must be serialised
 * by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_layer_forward_noalloc(const moe_layer *layer, const float *x, int T, float *y, const moe_route_io *route,
                              void *stream);

/* The same layer through the decode kernels with fp16 activations, for
 * 1 <= T <= 16 tokens in one pass: speed for accuracy, the trade the
 * strata-mlx engine offers between its 16-bit default and its slower,
 * exact float32 mode [strata-mlx wiki, "Measured"].  The expert FFN's
 * activations, x (normalised, for stacked layers)
 * and h = silu(g) u times the gate weight, are rounded to fp16 once instead
 * of being carried as fp16 hi + lo, so one matrix-core pass carries 16
 * tokens instead of 8 and every dequantized weight fragment serves twice as
 * many tokens; the router logits, the selection and the accumulation are
 * as in moe_layer_forward (the logits keep the hi + lo activations).
 * Arguments, routing input/output and errors as moe_layer_forward; T > 16 is
 * MOE_ERR_UNSUPPORTED.  ws_bytes >= moe_workspace_bytes(layer, T). */
int moe_layer_forward_f16act(const moe_layer *layer, const float *x, int T, float *y, const moe_route_io *route,
                             void *ws, size_t ws_bytes, void *stream);

/* A stack of layers with RMSNorm (unit weight) between consecutive layers
 * (T <= 16: decode kernels as in moe_layer_forward, the whole stack in one
 * pass; T > 16: prefill kernels, one layer after another):
 *   h_0 = x,  y_l = MoE_l(h_l),  h_{l+1} = y_l / sqrt(mean(y_l^2) + eps),
 *   y = y_{n-1}.
 * All layers must have equal d_model.  Optional per-layer outputs:
 *   y_layers   device fp32 [n][T][d] (every y_l), or NULL
 *   idx_layers device int32 [n][T][k], w_layers device fp32 [n][T][k], or NULL.
 * ws_bytes >= the largest moe_workspace_bytes over the layers. */
int moe_stack_forward(const moe_layer *const *layers, int n_layers, const float *x, int T, float eps,
                      float *y, float *y_layers, int32_t *idx_layers, float *w_layers, void *ws,
                      size_t ws_bytes, void *stream);

/* The stack through the decode kernels with fp16 activations (as
 * moe_layer_forward_f16act), 1 <= T <= 16 tokens per call, the whole stack
 * in one pass.  Arguments and outputs as moe_stack_forward; T > 16 is
 * MOE_ERR_UNSUPPORTED. */
int moe_stack_forward_f16act(const moe_layer *const *layers, int n_layers, const float *x, int T, float eps,
                             float *y, float *y_layers, int32_t *idx_layers, float *w_layers, void *ws,
                             size_t ws_bytes, void *stream);

/* Token-to-expert grouping (counting sort) of a routing idx device int32
 * [T][k].  Pair (t, r) names expert idx[t][r]; it is used unless that id is
 * outside [0, E) or repeats an earlier slot of the same token.  Outputs
 * (device int32):
 *   counts  [E]     used pairs per expert
 *   offsets [E+1]   exclusive prefix sum of counts; offsets[E] = used pairs
 *   perm    [T*k]   t*k + r of the used pairs, by expert ascending and token
 *                   ascending within an expert, then -1 up to T*k
 * Bit-exact with the plain definition.  ws: device scratch of at least
 * moe_group_workspace_bytes(T, E, k) bytes, 256-byte aligned.  This is the
 * step the prefill path runs before its grouped matrix multiply.
 * 0 <= T <= 65536, 1 <= E <= 4096, 1 <= k <= 16. */
int moe_group_workspace_bytes(int T, int E, int k, size_t *bytes);
int moe_group_tokens(const int32_t *idx, int T, int E, int k, int32_t *counts, int32_t *offsets, int32_t *perm,
                     void *ws, size_t ws_bytes, void *stream);

/* y[t] = x[t] / sqrt(mean(x[t]^2) + eps), fp32 in and out, d % 4 == 0. */
int moe_rmsnorm(const float *x, int T, int d, float eps, float *y, void *stream);

/* Test export of device-decoded weights of one matrix of one expert
 * (expert = -1: shared expert; mat 0 = gate, 1 = up, 2 = down), read back
 * from the packed layout:
 *   codes  device int8 [rows][cols] signed codes, or NULL
 *   w_f32  device fp32 [rows][cols] scale * code (exact), or NULL
 *   w_f16  device uint16 [rows][cols] fp16 bits of scale * code (round to
 *          nearest even; exact for 2-bit codes), or NULL
 * rows x cols is [I][d] for gate/up and [d][I] for down. */
int moe_debug_unpack(const moe_layer *layer, int expert, int mat, int8_t *codes, float *w_f32,
                     uint16_t *w_f16, void *stream);

/* Test export of the same matrix through the decoders the expert kernels run
 * (moe_debug_unpack above has a decoder of its own), so that the weights the
 * multiplications actually see can be compared bit for bit:
 *   path 0  the decode kernels' fragment decode: codes come out of the packed
 *           chunk as exact fp16 integers (the matrix-core B operand) and the
 *           fp16 block scale as the epilogue factor; exports codes (int8,
 *           q - 2^(b-1)) and/or w_f32 = scale * code; w_f16 must be NULL;
 *   path 1  the grouped GEMMs' register dequantization from half chunks (the
 *           gate/up kernel's loads): exports w_f16, the fp16 bits of
 *           scale * code rounded once to nearest even; codes and w_f32 must
 *           be NULL;
 *   path 2  the same dequantization from whole chunks (the down kernel's
 *           loads when a chunk holds 4 or 2 blocks of a row).
 * Layouts and errors as moe_debug_unpack; a bad path is MOE_ERR_ARG. */
int moe_debug_unpack_path(const moe_layer *layer, int expert, int mat, int path, int8_t *codes, float *w_f32,
                          uint16_t *w_f16, void *stream);

/* Status of the last persistent decode pass that used this workspace: 0 = it
 * ran to completion; 1 = it gave up.  The decode kernels of a layer or stack
 * of layers of one shape (at most 1024 experts) run as one persistent kernel
 * whose workgroups (one per compute unit) hand results to each other; every
 * wait in it is bounded, and a pass that cannot make progress (its
 * workgroups are not all resident at once, e.g. because other work occupies
 * the device) ends early with unspecified outputs and this status set.  The
 * status stays until the next pass on the workspace.  This call waits for
 * `stream`. */
int moe_workspace_status(const void *ws, size_t ws_bytes, int *status, void *stream);

/* Tuning overrides read from the environment at each call (set them before
 * the first call and leave them unchanged: the split count also sets the
 * workspace layout, so moe_workspace_bytes and the forward calls must see
 * the same value).  Defaults in brackets.
 *   MOE_GU_WGS       decode gate/up workgroups [the CU count, at most the
 *                    number of 16-row tiles]
 *   MOE_GU_SHARED_WGS  of those, the workgroups that run only the shared
 *                    expert's items, starting without the selection [one
 *                    per four of its 16-row tiles; 0 = every workgroup
 *                    selects and takes a share of all items]
 *   MOE_DOWN_SPLITS  decode down-projection splits [2 x CUs / row groups,
 *                    clamped to 1..8 and to the slot count]
 *   MOE_DOWN_WAVES   wavefronts per decode down workgroup [8; 1..8]
 *   MOE_PERSIST      1 = run a stack of layers of one shape (at most 1024
 *                    experts) as one persistent launch per 16 layers; 0 =
 *                    separate kernels per layer (route, gate/up, down) [0]
 *                    (up to 8 tokens and the fp16-activation calls only)
 *   MOE_MID_T        1 = 9..16 tokens through one decode pass of 16 hi + lo
 *                    token rows; 0 = a layer through the chunked-prefill
 *                    kernels, a stack in decode passes of 8 tokens [1] */

/* Per-kernel timing for measurement: while enabled, the library brackets
 * every launch of the chosen kernel class with a pair of HIP events that the
 * launch records itself (the start and end of its dispatch), and every
 * kernel of the layer functions waits for the stream to drain on the host
 * first, so each runs alone (it must not be enabled while a graph is being
 * captured).  class 0 = decode gate/up expert kernel, 1 = decode down
 * expert kernel, 2 = decode router, 3 = prefill gate/up grouped GEMM, 4 =
 * prefill down grouped GEMM, 5 = prefill router GEMM, 6 = persistent decode
 * pass (one launch per pass of up to 64 layers).  moe_timing_stop waits
 * for the recorded events and returns the summed duration and the number of
 * launches. */
int moe_timing_start(int kernel_class, int max_launches);
int moe_timing_stop(double *total_ms, int *launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
