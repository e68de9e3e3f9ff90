/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU model of the low-bit sparse
 * mixture-of-experts layer, written to check the HIP path against.  Every
 * quantity is computed in fp64 with scalar loops in the order the method
 * states; nothing here is blocked, fused or vectorised by hand.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load this library; the product path never does.
 *
 * What the method computes (sources are the five pages; no page writes the
 * layer as equations, so the steps below are the plain reading of them):
 *   - experts stay in their low-bit blocks and are multiplied from them
 *     [strata-mlx wiki, opening feature list, first item; devlabs blog
 *     "32GB Mac mini 6 ...", section 核心技术特点];
 *   - a router picks about ten of 512 small experts per token, next to an
 *     always-used shared expert [cnyes profile of Strata, sections
 *     "Strata 到底是什麼？" and "三層記憶體" part 1];
 *   - block unpacking follows the ggml block types [strata-mlx wiki, credits
 *     list, llama.cpp/ggml entry].
 *
 * Readings taken where the pages are silent:
 *   R1 block = {fp16 scale, 32 codes of b bits}; code j occupies bits
 *      [b*j, b*j+b) of the little-endian bitstream formed by the code bytes.
 *   R2 signed code c = q - 2^(b-1) (offset binary).
 *   R3 gate/up are [I][d], down is [d][I], row-major, blocks along the
 *      input dimension of each matrix.
 *   R4 top-k on fp32 logits, order (logit descending, index ascending);
 *      gate weights = softmax over the k selected logits, computed with the
 *      deterministic exp64 below.
 *   R5 shared expert has weight 1 and no gate.
 *   R6 stack glue = RMSNorm with unit weight and eps 1e-6 between layers.
 *   R7 codebook blocks (the codebook block types the same credits list
 *      names, whose tables ship with the model file and are absent here, so
 *      a synthetic table of the same shape stands in): 32 weights per block,
 *      15 bytes: [0,2) fp16 scale; [2,10) the low 8 bits of eight 9-bit
 *      grid indices, index i covering weights 4i..4i+3; byte 10, bit i = bit
 *      8 of index i; [11,15) 32 sign bits, bit j of the little-endian word
 *      set = weight j negative.  Weight j = scale * (+-1) * G[index][j % 4]
 *      for a grid G of 512 entries of 4 unsigned magnitudes (0..127).
 *   R8 a forced routing row names each expert at most once: an entry
 *      outside [0, E) or repeating an expert of an earlier rank of the same
 *      token contributes nothing (the same rule as the token grouping).
 *
 * Every function here is pinned by a CPU test (values fixed by the
 * mathematics, brute force, closed forms and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_MISSING_EXPERT (-2)
#define ORC_ERR_NONFINITE (-3)

/* ------------------------------------------------------------------ */
/* fp16 <-> fp64, from the IEEE 754 binary16 layout: 1 sign bit,        */
/* 5 exponent bits (bias 15), 10 fraction bits.                         */
/* ------------------------------------------------------------------ */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + f/1024) 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even, and return
 * its bit pattern.  Overflow goes to infinity; NaN maps to 0x7e00. */
uint16_t orc_double_to_half(double v)
{
    uint16_t sign = 0;
    if (isnan(v)) return 0x7e00;
    if (signbit(v)) { sign = 0x8000; v = -v; }
    if (isinf(v)) return sign | 0x7c00;
    if (v == 0.0) return sign;
    int e;
    frexp(v, &e);            /* v = m * 2^e, m in [0.5, 1) */
    int expo = e - 1;        /* v in [2^expo, 2^(expo+1)) */
    /* quantum of the binary16 grid at this magnitude */
    int qexp = (expo < -14) ? -24 : expo - 10;
    double n = v / ldexp(1.0, qexp);          /* exact: power-of-two scale */
    double fl = floor(n);
    double rem = n - fl;                       /* exact */
    double r;
    if (rem > 0.5) r = fl + 1.0;
    else if (rem < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double q = r * ldexp(1.0, qexp);
    if (q > 65504.0) return sign | 0x7c00;
    /* re-encode the exact binary16 value q */
    if (q < ldexp(1.0, -14)) {
        return sign | (uint16_t)(q / ldexp(1.0, -24));
    }
    int qe;
    frexp(q, &qe);
    int be = qe - 1;                            /* q in [2^be, 2^(be+1)) */
    uint16_t fr = (uint16_t)((q / ldexp(1.0, be) - 1.0) * 1024.0);
    return sign | (uint16_t)((be + 15) << 10) | fr;
}

/* Array form of orc_double_to_half. */
void orc_double_to_half_array(const double *v, long n, uint16_t *out)
{
    for (long i = 0; i < n; ++i) out[i] = orc_double_to_half(v[i]);
}

/* ------------------------------------------------------------------ */
/* Canonical block: bytes [0,2) fp16 scale (little endian), then 4*b     */
/* bytes of codes.  Readings R1, R2.                                     */
/* ------------------------------------------------------------------ */
int orc_block_bytes(int bits) { return 2 + 4 * bits; }

/* Unpack one block: 32 signed codes and the scale as fp64. */
void orc_unpack_block(const uint8_t *blk, int bits, int8_t *codes, double *scale)
{
    uint16_t sbits = (uint16_t)(blk[0] | (blk[1] << 8));
    const uint8_t *q = blk + 2;
    for (int j = 0; j < 32; ++j) {
        int val = 0;
        for (int i = 0; i < bits; ++i) {
            int pos = bits * j + i;
            int bit = (q[pos >> 3] >> (pos & 7)) & 1;
            val |= bit << i;
        }
        codes[j] = (int8_t)(val - (1 << (bits - 1)));
    }
    *scale = orc_half_to_double(sbits);
}

/* Unpack a whole canonical matrix [rows][cols] (cols % 32 == 0):
 * codes[rows*cols], scales[rows*(cols/32)] as fp64. */
int orc_unpack_matrix(const uint8_t *canon, int rows, int cols, int bits,
                      int8_t *codes, double *scales)
{
    if (cols % 32 || rows < 0 || (bits != 2 && bits != 3)) return ORC_ERR_ARG;
    int nb = cols / 32, bb = orc_block_bytes(bits);
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b) {
            const uint8_t *blk = canon + ((size_t)r * nb + b) * bb;
            orc_unpack_block(blk, bits, codes + (size_t)r * cols + 32 * b,
                             scales + (size_t)r * nb + b);
        }
    return ORC_OK;
}

/* Dequantised weights w = scale * code, fp64 (exact: an fp16 value times an
 * integer of magnitude <= 4 has at most 14 significant bits). */
int orc_dequant_matrix(const uint8_t *canon, int rows, int cols, int bits, double *w)
{
    if (cols % 32 || rows < 0 || (bits != 2 && bits != 3)) return ORC_ERR_ARG;
    int nb = cols / 32, bb = orc_block_bytes(bits);
    int8_t c[32];
    double s;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b) {
            orc_unpack_block(canon + ((size_t)r * nb + b) * bb, bits, c, &s);
            for (int j = 0; j < 32; ++j)
                w[(size_t)r * cols + 32 * b + j] = s * (double)c[j];
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Codebook block (reading R7): 15 bytes, 32 weights.                    */
/* ------------------------------------------------------------------ */
#define ORC_CB_BLOCK_BYTES 15
#define ORC_CB_ENTRIES 512
int orc_cb_block_bytes(void) { return ORC_CB_BLOCK_BYTES; }

/* Unpack one codebook block: 32 signed codes (the looked-up magnitude with
 * the block's sign bit applied) and the scale as fp64.  grid is [512][4]. */
void orc_cb_unpack_block(const uint8_t *blk, const uint8_t *grid, int8_t *codes, double *scale)
{
    uint16_t sbits = (uint16_t)(blk[0] | (blk[1] << 8));
    uint32_t signs = (uint32_t)blk[11] | ((uint32_t)blk[12] << 8) |
                     ((uint32_t)blk[13] << 16) | ((uint32_t)blk[14] << 24);
    for (int i = 0; i < 8; ++i) {
        int index = blk[2 + i] | (((blk[10] >> i) & 1) << 8);
        for (int c = 0; c < 4; ++c) {
            int j = 4 * i + c;
            int m = grid[4 * index + c];
            codes[j] = (int8_t)(((signs >> j) & 1) ? -m : m);
        }
    }
    *scale = orc_half_to_double(sbits);
}

static int grid_ok(const uint8_t *grid)
{
    if (!grid) return 0;
    for (int i = 0; i < 4 * ORC_CB_ENTRIES; ++i)
        if (grid[i] > 127) return 0;
    return 1;
}

/* Whole canonical codebook matrix [rows][cols]: codes[rows*cols],
 * scales[rows*(cols/32)]. */
int orc_cb_unpack_matrix(const uint8_t *canon, int rows, int cols, const uint8_t *grid,
                         int8_t *codes, double *scales)
{
    if (cols % 32 || rows < 0 || !grid_ok(grid)) return ORC_ERR_ARG;
    int nb = cols / 32;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b)
            orc_cb_unpack_block(canon + ((size_t)r * nb + b) * ORC_CB_BLOCK_BYTES, grid,
                                codes + (size_t)r * cols + 32 * b, scales + (size_t)r * nb + b);
    return ORC_OK;
}

/* w = scale * code in fp64 (exact: 11 significant bits times a magnitude
 * below 128, at most 18 bits, so exact in fp32 too). */
int orc_cb_dequant_matrix(const uint8_t *canon, int rows, int cols, const uint8_t *grid, double *w)
{
    if (cols % 32 || rows < 0 || !grid_ok(grid)) return ORC_ERR_ARG;
    int nb = cols / 32;
    int8_t c[32];
    double s;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b) {
            orc_cb_unpack_block(canon + ((size_t)r * nb + b) * ORC_CB_BLOCK_BYTES, grid, c, &s);
            for (int j = 0; j < 32; ++j)
                w[(size_t)r * cols + 32 * b + j] = s * (double)c[j];
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* exp64: deterministic fp64 exponential, written from the mathematics   */
/* so that any implementation following the same steps in IEEE fp64     */
/* reproduces it bit for bit:                                            */
/*   n = rint(z / ln 2), r = z - n ln 2 (two fused steps, ln 2 split in  */
/*   a high and a low part), p = sum_{i<=13} r^i / i! by Horner with     */
/*   fused multiply-add, result = p * 2^n.                                */
/* |r| <= ln2/2, so the Taylor remainder is below 2^-60 relative.         */
/* The constants are the fp64 values nearest to 1/i! and to ln 2.        */
/* ------------------------------------------------------------------ */
static const double ORC_INV_LN2 = 0x1.71547652b82fep+0;   /* nearest to 1/ln2 */
static const double ORC_LN2_HI = 0x1.62e42fefa39efp-1;    /* nearest to ln2 */
static const double ORC_LN2_LO = 0x1.abc9e3b39803fp-56;   /* nearest to ln2 - LN2_HI */
static const double ORC_INV_FACT[14] = {
    0x1p+0,                 /* 1/0!  */
    0x1p+0,                 /* 1/1!  */
    0x1p-1,                 /* 1/2!  */
    0x1.5555555555555p-3,   /* 1/3!  */
    0x1.5555555555555p-5,   /* 1/4!  */
    0x1.1111111111111p-7,   /* 1/5!  */
    0x1.6c16c16c16c17p-10,  /* 1/6!  */
    0x1.a01a01a01a01ap-13,  /* 1/7!  */
    0x1.a01a01a01a01ap-16,  /* 1/8!  */
    0x1.71de3a556c734p-19,  /* 1/9!  */
    0x1.27e4fb7789f5cp-22,  /* 1/10! */
    0x1.ae64567f544e4p-26,  /* 1/11! */
    0x1.1eed8eff8d898p-29,  /* 1/12! */
    0x1.6124613a86d09p-33,  /* 1/13! */
};

double orc_exp64(double z)
{
    if (z < -1080.0) return 0.0;   /* below the smallest subnormal */
    if (z > 709.0) return INFINITY;
    double n = rint(z * ORC_INV_LN2);
    double r = fma(-n, ORC_LN2_HI, z);
    r = fma(-n, ORC_LN2_LO, r);
    double p = ORC_INV_FACT[13];
    for (int i = 12; i >= 0; --i) p = fma(p, r, ORC_INV_FACT[i]);
    return ldexp(p, (int)n);
}

/* Coefficient tables exposed for pinning against exact rationals. */
double orc_exp64_coeff(int i) { return (i >= 0 && i < 14) ? ORC_INV_FACT[i] : NAN; }
double orc_exp64_ln2(int part) { return part == 0 ? ORC_LN2_HI : part == 1 ? ORC_LN2_LO : ORC_INV_LN2; }

/* ------------------------------------------------------------------ */
/* Router: logit[t][e] = fp32( sum_j x[t][j] W[e][j] (fp64, j ascending)  */
/*                             + bias[e] ).                              */
/* Source: the router that picks ~10 of 512 experts per token [cnyes     */
/* profile, section "Strata 到底是什麼？"]; a linear router with bias is   */
/* the plain reading.                                                    */
/* ------------------------------------------------------------------ */
void orc_router_logits(const float *x, const float *W, const float *bias,
                       int T, int d, int E, float *logits)
{
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += (double)x[(size_t)t * d + j] * (double)W[(size_t)e * d + j];
            if (bias) acc += (double)bias[e];
            logits[(size_t)t * E + e] = (float)acc;
        }
}

/* ------------------------------------------------------------------ */
/* Top-k selection + gate weights (reading R4).                          */
/* Rank r is the not-yet-taken expert with the largest logit; among      */
/* equal logits the lowest index wins (strict '>' while scanning upward). */
/* Gate weights: m = logit of rank 0, e_r = exp64(l_r - m),               */
/* S = sum of e_r in rank order, w_r = fp32(e_r / S).                     */
/* Returns ORC_ERR_NONFINITE if a logit is not finite.                    */
/* ------------------------------------------------------------------ */
int orc_topk(const float *logits, int T, int E, int k, int32_t *idx, float *w)
{
    if (k < 1 || k > E) return ORC_ERR_ARG;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *ev = (double *)malloc(sizeof(double) * (size_t)k);
    if (!taken || !ev) { free(taken); free(ev); return ORC_ERR_ARG; }
    int rc = ORC_OK;
    for (int t = 0; t < T && rc == ORC_OK; ++t) {
        const float *l = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e)
            if (!isfinite(l[e])) rc = ORC_ERR_NONFINITE;
        memset(taken, 0, (size_t)E);
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * k + r] = best;
        }
        double m = (double)l[idx[(size_t)t * k]];
        double S = 0.0;
        for (int r = 0; r < k; ++r) {
            ev[r] = orc_exp64((double)l[idx[(size_t)t * k + r]] - m);
            S += ev[r];
        }
        for (int r = 0; r < k; ++r) w[(size_t)t * k + r] = (float)(ev[r] / S);
    }
    free(taken);
    free(ev);
    return rc;
}

/* ------------------------------------------------------------------ */
/* One expert, SwiGLU feed-forward from canonical blocks (reading R3):    */
/*   g_i = sum_j Wg[i][j] x_j,  u_i = sum_j Wu[i][j] x_j,                 */
/*   h_i = silu(g_i) u_i,  silu(z) = z / (1 + exp(-z)),                   */
/*   y_o = sum_i Wd[o][i] h_i.                                            */
/* All sums in fp64, ascending index; weights dequantised block by block. */
/* Expert canonical bytes: gate [I][d/32 blocks], up [I][d/32], down      */
/* [d][I/32], consecutive.                                                */
/* ------------------------------------------------------------------ */
/* A block of either format: plain b-bit codes, or codebook blocks when a
 * grid is given. */
static int any_block_bytes(int bits, const uint8_t *grid)
{
    return grid ? ORC_CB_BLOCK_BYTES : orc_block_bytes(bits);
}

static double matvec_row(const uint8_t *row_blocks, int cols, int bits, const uint8_t *grid, const double *v)
{
    int bb = any_block_bytes(bits, grid);
    int8_t c[32];
    double s, acc = 0.0;
    for (int b = 0; b < cols / 32; ++b) {
        if (grid) orc_cb_unpack_block(row_blocks + (size_t)b * bb, grid, c, &s);
        else orc_unpack_block(row_blocks + (size_t)b * bb, bits, c, &s);
        for (int j = 0; j < 32; ++j) acc += (s * (double)c[j]) * v[32 * b + j];
    }
    return acc;
}

size_t orc_expert_bytes(int d, int I, int bits)
{
    return (size_t)3 * (size_t)I * (size_t)(d / 32) * (size_t)orc_block_bytes(bits);
}

size_t orc_cb_expert_bytes(int d, int I)
{
    return (size_t)3 * (size_t)I * (size_t)(d / 32) * (size_t)ORC_CB_BLOCK_BYTES;
}

/* The expert FFN from blocks of either format (grid NULL: b-bit blocks). */
int orc_expert_ffn_any(const uint8_t *ex, int d, int I, int bits, const uint8_t *grid,
                       const double *x, double *y)
{
    if (d % 32 || I % 32) return ORC_ERR_ARG;
    if (grid ? !grid_ok(grid) : (bits != 2 && bits != 3)) return ORC_ERR_ARG;
    int bb = any_block_bytes(bits, grid);
    size_t gate_row = (size_t)(d / 32) * bb, down_row = (size_t)(I / 32) * bb;
    const uint8_t *Wg = ex, *Wu = ex + (size_t)I * gate_row, *Wd = ex + 2 * (size_t)I * gate_row;
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    if (!h) return ORC_ERR_ARG;
    for (int i = 0; i < I; ++i) {
        double g = matvec_row(Wg + (size_t)i * gate_row, d, bits, grid, x);
        double u = matvec_row(Wu + (size_t)i * gate_row, d, bits, grid, x);
        h[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int o = 0; o < d; ++o) y[o] = matvec_row(Wd + (size_t)o * down_row, I, bits, grid, h);
    free(h);
    return ORC_OK;
}

int orc_expert_ffn(const uint8_t *ex, int d, int I, int bits, const double *x, double *y)
{
    return orc_expert_ffn_any(ex, d, I, bits, NULL, x, y);
}

/* ------------------------------------------------------------------ */
/* Layer forward.                                                        */
/* ------------------------------------------------------------------ */
typedef struct {
    int d, E, I, Is, k, bits;
    const float *router_w;      /* [E][d] */
    const float *router_bias;   /* [E] or NULL (= 0) */
    const uint8_t *const *experts; /* E pointers; NULL for experts never selected */
    const uint8_t *shared;      /* shared expert canonical bytes, NULL if Is == 0 */
    const uint8_t *grid;        /* codebook [512][4] for codebook blocks, NULL for b-bit blocks */
} orc_layer;

/* y[t] = fp32( sum_{r in rank order} w[t][r] * FFN_{idx[t][r]}(x[t])
 *              + FFN_shared(x[t]) ), one rounding at the end.
 * force_idx/force_w (both or neither) replace the router's choice, which
 * is how the GPU's own routing is fed in for a teacher-forced check.
 * logits_out / idx_out / w_out may be NULL. */
int orc_layer_forward(const orc_layer *L, const float *x, int T,
                      const int32_t *force_idx, const float *force_w,
                      float *logits_out, int32_t *idx_out, float *w_out, float *y)
{
    int d = L->d, E = L->E, k = L->k, rc = ORC_OK;
    if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E) return ORC_ERR_ARG;
    if ((force_idx == NULL) != (force_w == NULL)) return ORC_ERR_ARG;
    if (T == 0) return ORC_OK;
    float *logits = (float *)malloc(sizeof(float) * (size_t)T * E);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
    float *w = (float *)malloc(sizeof(float) * (size_t)T * k);
    double *xv = (double *)malloc(sizeof(double) * (size_t)d);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    double *ye = (double *)malloc(sizeof(double) * (size_t)d);
    if (!logits || !idx || !w || !xv || !acc || !ye) { rc = ORC_ERR_ARG; goto out; }

    if (force_idx) {
        memcpy(idx, force_idx, sizeof(int32_t) * (size_t)T * k);
        memcpy(w, force_w, sizeof(float) * (size_t)T * k);
        if (logits_out) orc_router_logits(x, L->router_w, L->router_bias, T, d, E, logits);
    } else {
        orc_router_logits(x, L->router_w, L->router_bias, T, d, E, logits);
        rc = orc_topk(logits, T, E, k, idx, w);
        if (rc != ORC_OK) goto out;
    }
    for (int t = 0; t < T && rc == ORC_OK; ++t) {
        for (int j = 0; j < d; ++j) { xv[j] = (double)x[(size_t)t * d + j]; acc[j] = 0.0; }
        for (int r = 0; r < k; ++r) {
            int e = idx[(size_t)t * k + r];
            if (e < 0 || e >= E) continue;  /* reading R8 */
            int earlier = 0;
            for (int q = 0; q < r; ++q) earlier |= idx[(size_t)t * k + q] == e;
            if (earlier) continue;
            if (!L->experts || !L->experts[e]) { rc = ORC_ERR_MISSING_EXPERT; break; }
            rc = orc_expert_ffn_any(L->experts[e], d, L->I, L->bits, L->grid, xv, ye);
            if (rc != ORC_OK) break;
            double g = (double)w[(size_t)t * k + r];
            for (int o = 0; o < d; ++o) acc[o] += g * ye[o];
        }
        if (rc != ORC_OK) break;
        if (L->Is > 0) {
            if (!L->shared) { rc = ORC_ERR_MISSING_EXPERT; break; }
            rc = orc_expert_ffn_any(L->shared, d, L->Is, L->bits, L->grid, xv, ye);
            if (rc != ORC_OK) break;
            for (int o = 0; o < d; ++o) acc[o] += ye[o];
        }
        for (int o = 0; o < d; ++o) y[(size_t)t * d + o] = (float)acc[o];
    }
    if (rc == ORC_OK) {
        if (logits_out) memcpy(logits_out, logits, sizeof(float) * (size_t)T * E);
        if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)T * k);
        if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)T * k);
    }
out:
    free(logits); free(idx); free(w); free(xv); free(acc); free(ye);
    return rc;
}

/* RMSNorm with unit weight between stacked layers (reading R6):
 * y = fp32( x / sqrt(mean(x^2) + eps) ), mean in fp64. */
void orc_rmsnorm(const float *x, int T, int d, double eps, float *y)
{
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int j = 0; j < d; ++j) {
            double v = (double)x[(size_t)t * d + j];
            ss += v * v;
        }
        double den = sqrt(ss / (double)d + eps);
        for (int j = 0; j < d; ++j) y[(size_t)t * d + j] = (float)((double)x[(size_t)t * d + j] / den);
    }
}

/* Grouping of (token, slot) pairs by expert: the token-to-expert counting
 * sort that precedes the per-expert matrix products when many tokens are
 * processed at once (prompt chunks of up to 8192 tokens [agentlenshq
 * article, section "Strata 如何让 125 B 模型适配 12-24 GB 显存", last
 * item]).  Pair (t, r) names expert idx[t][r]; it is used unless that id is
 * outside [0, E) or repeats an id of an earlier slot of the same token.
 *   counts[e]    number of used pairs naming e
 *   offsets[e]   sum of counts of experts below e; offsets[E] = all used pairs
 *   perm[j]      t*k + r of the used pairs, by expert ascending, and by token
 *                ascending within one expert; -1 after offsets[E]
 * Plain definition, one pass per expert. */
void orc_group_tokens(const int32_t *idx, int T, int E, int k,
                      int32_t *counts, int32_t *offsets, int32_t *perm)
{
    long n = (long)T * k, pos = 0;
    for (long j = 0; j < n; ++j) perm[j] = -1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int32_t c = 0;
        for (int t = 0; t < T; ++t) {
            for (int r = 0; r < k; ++r) {
                if (idx[(long)t * k + r] != e) continue;
                int earlier = 0;
                for (int q = 0; q < r; ++q) earlier |= idx[(long)t * k + q] == e;
                if (earlier) continue;
                perm[pos++] = (int32_t)((long)t * k + r);
                ++c;
            }
        }
        counts[e] = c;
        offsets[e + 1] = offsets[e] + c;
    }
}
