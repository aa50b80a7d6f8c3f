/*
 * moe_oracle.c - plain, slow, fp64 CPU oracle for the sparse mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls this file: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg do. It shares no code,
 * header, table or helper with the HIP library; both sides read the same stored input values.
 *
 * Sources (the pages are cited by title; they have no numbered sections):
 *   [PR8]  "feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8" (ninfer-windows pull
 *          request #8), the commit message on the small-T MoE router: the S1/S2 description,
 *          the "two changes" list, the paragraph explaining why the output is bit-identical,
 *          and the paragraph on the double-precision CPU reference.
 *   [REL09] "RELEASE_NOTES_0.9.0" of the 16 GB ninfer fork: the MoE share of the weights and the
 *          bandwidth-bound decode paragraph (experts are streamed once per token).
 *   The layer definition (router GEMV with a shared-expert gate row, top-8, softmax over the
 *   selected eight, sigmoid shared gate, SwiGLU experts, weighted sum) is the plain reading of
 *   those passages; every reading taken where the pages are silent is listed in the design notes.
 *
 * What each function computes, in the plainest form:
 *   oracle_logits   z[t][r] = fp32( sum_h W[r][h] * x[t][h] + b[r] ), accumulated in fp64 and rounded
 *                   once. The router has one row per expert plus, when a shared expert exists, one
 *                   more row whose score is the shared-expert gate logit ([PR8]: a 257-entry score
 *                   array per token next to the shared-expert sigmoid).
 *   oracle_select   eight rounds of argmax under the total order of [PR8] (greater value first, the
 *                   lower expert id on equal values), each round excluding the experts already
 *                   taken; then the softmax over the eight selected logits and the sigmoid of the
 *                   gate logit, both in fp64. This is the old selection loop's algorithm; [PR8]
 *                   states that the order is total, so the result is unique and any exact method
 *                   (the merge network included) must return the same ids in the same order.
 *   oracle_bucket   a stable counting sort of the (token, rank) pairs by expert id.
 *   oracle_forward  for each requested token: sum over the eight ranks of w_k * FFN_{id_k}(x) plus
 *                   g * FFN_shared(x), where FFN(x) = Wd (silu(Wg x) * (Wu x)) and
 *                   silu(a) = a / (1 + exp(-a)); every step in fp64 with no intermediate rounding.
 *   oracle_forward_w the same with quantized expert weights, each weight's value taken exactly in
 *                   fp64 before the products: FP8 - its E4M3 code's value times its row's fp32
 *                   scale; MXFP4 - its E2M1 code's value times the E8M0 scale of its block of 32
 *                   consecutive weights along the row (the pages name quantized expert formats -
 *                   groupwise integers, FP8, NVFP4 - without fixing one; these two, per-row-scaled
 *                   E4M3 and the Open Compute Project's MXFP4, are the readings here).
 *
 * Comparison semantics: IEEE-754 fp32 values compared as values, so -0 equals +0 (a tie, decided
 * by the id). NaN ranks below every non-NaN value, -inf included; NaNs tie among themselves and
 * the lower id wins. (The pages say nothing about signed zeros or NaN; these are the readings.)
 *
 * ORACLE_PLANT_* macros build deliberately wrong variants (CPU only) so that the tests can show
 * each pin rejects a plausible mistake; the normal build defines none of them.
 *
 * Parity pins live in the CPU test suite: brute-force full sort, closed forms, integer-exact
 * logits, and a numpy SwiGLU; see tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_FP8 2 /* weights only: OCP FP8 E4M3 codes, each row times its own fp32 scale */
#define ORACLE_MXFP4 3 /* weights only: OCP MXFP4 - E2M1 codes, two per byte (the even column in
                          the low nibble), each block of 32 columns times its E8M0 scale byte */
#define MX_BLOCK 32    /* weights per shared scale in MXFP4 */

/* Value of one OCP FP8 E4M3 code (the 8-bit floating-point format of the Open Compute Project
 * specification: sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, and
 * S.1111.111 is NaN). Exponent field 0 holds the subnormals m * 2^-9; otherwise the value is
 * 2^(e - 7) * (1 + m / 8). Exact in double. */
double oracle_e4m3_value(uint8_t code) {
    const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
#ifdef ORACLE_PLANT_E4M3_BIAS8
    if (e == 0) v = ldexp((double)m, -10); /* planted mistake: the other FP8 family's bias 8 */
    else v = ldexp(1.0 + m / 8.0, e - 8);
#else
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
#endif
    return s ? -v : v;
}

/* Value of one FP4 E2M1 code (the 4-bit element type of the Open Compute Project's Microscaling
 * (MX) formats specification): sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent
 * field 0 holds zero and the subnormal 0.5, otherwise the value is 2^(e - 1) * (1 + m / 2). No
 * infinities or NaN: the eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. Exact in double. */
double oracle_e2m1_value(uint8_t code) {
    const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
#ifdef ORACLE_PLANT_E2M1_BIAS2
    const double v = e == 0 ? 0.25 * m : ldexp(1.0 + 0.5 * m, e - 2); /* planted: bias 2 */
#else
    const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
#endif
    return s ? -v : v;
}

/* Value of one E8M0 scale byte (the MX formats' shared scale: an unsigned exponent with bias 127
 * and no mantissa): 2^(b - 127); the byte 0xFF is NaN. Exact in double. */
double oracle_e8m0_value(uint8_t b) {
    if (b == 0xFF) return NAN;
#ifdef ORACLE_PLANT_E8M0_BIAS128
    return ldexp(1.0, (int)b - 128); /* planted mistake: bias off by one */
#else
    return ldexp(1.0, (int)b - 127);
#endif
}

/* Widen one stored element to double. bf16 is the top half of an fp32 word, so the value is the
 * 16 stored bits shifted into the high half; the conversion is exact. An FP8 element is its
 * code's value times the fp32 scale of its row (given by the caller). */
static inline __attribute__((always_inline)) double load_elem(const void *base, int dtype, size_t i) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[i];
    if (dtype == ORACLE_FP8) return oracle_e4m3_value(((const uint8_t *)base)[i]);
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t elem_size(int dtype) {
    return dtype == ORACLE_F32 ? 4 : dtype == ORACLE_FP8 ? 1 : 2;
}

/* Weight (row, col) of a matrix with `cols` columns in weight format wdtype, as a double, with
 * the scales of row srow (always row itself, except in one planted-mistake build). FP8: the
 * code's value times the row's fp32 scale (scale[srow]; 1 without scales). MXFP4: codes packed
 * two per byte along the row (column 2j in the low nibble of byte j, 2j + 1 in the high one),
 * scale bytes [rows][cols / 32]; the weight is the code's value times its block's scale. */
static inline __attribute__((always_inline)) double weight_at(const void *m, const void *scale,
                                                               int wdtype, int row, int col,
                                                               int cols, int srow) {
    if (wdtype == ORACLE_MXFP4) {
        const uint8_t b = ((const uint8_t *)m)[(size_t)row * (cols / 2) + col / 2];
#ifdef ORACLE_PLANT_FP4_HIGH_FIRST
        const uint8_t code = (col & 1) ? (b & 15) : (b >> 4); /* planted: nibble order swapped */
#else
        const uint8_t code = (col & 1) ? (b >> 4) : (b & 15);
#endif
        const uint8_t sb = ((const uint8_t *)scale)[(size_t)srow * (cols / MX_BLOCK) + col / MX_BLOCK];
        return oracle_e2m1_value(code) * oracle_e8m0_value(sb);
    }
    const double v = load_elem(m, wdtype, (size_t)row * cols + col);
    if (wdtype == ORACLE_FP8 && scale) return v * (double)((const float *)scale)[srow];
    return v;
}

/* Bytes of one stored [rows][cols] weight matrix, and of its scales (0 without). */
static size_t matrix_bytes(int wdtype, int rows, int cols) {
    if (wdtype == ORACLE_MXFP4) return (size_t)rows * (cols / 2);
    return (size_t)rows * cols * elem_size(wdtype);
}
static size_t scale_bytes(int wdtype, int rows, int cols) {
    if (wdtype == ORACLE_FP8) return (size_t)rows * sizeof(float);
    if (wdtype == ORACLE_MXFP4) return (size_t)rows * (cols / MX_BLOCK);
    return 0;
}

/* ---------------------------------------------------------------- router logits */
int oracle_logits(int T, int H, int R, int dtype, const void *x, const void *W, const float *bias,
                  float *z_out) {
    if (T < 0 || H <= 0 || R <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += load_elem(W, dtype, (size_t)r * H + h) * load_elem(x, dtype, (size_t)t * H + h);
#ifndef ORACLE_PLANT_DROP_BIAS
            if (bias) acc += (double)bias[r];
#endif
            z_out[(size_t)t * R + r] = (float)acc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- the total order */
/* 1 iff expert a (value va) ranks strictly above expert b (value vb). */
static int ranks_above(float va, int a, float vb, int b) {
    int na = isnan(va), nb = isnan(vb);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb; /* the non-NaN one is above */
    }
    if (va > vb) return 1;
    if (va < vb) return 0;
#ifdef ORACLE_PLANT_TIE_HIGH_ID
    return a > b; /* planted mistake: the higher id wins ties */
#else
    return a < b; /* equal values (this includes -0 == +0): the lower id wins */
#endif
}

/* ---------------------------------------------------------------- top-k, softmax, gate */
/* z: [T][stride] fp32; experts are columns 0..E-1; when has_gate, column E is the gate logit.
 * ids: [T][k] int32, w: [T][k] fp64, g: [T] fp64 (written only when has_gate). */
int oracle_select(int T, int E, int stride, const float *z, int has_gate, int k, int32_t *ids,
                  double *w, double *g) {
    if (T < 0 || E <= 0 || k <= 0 || k > E || stride < E + (has_gate ? 1 : 0)) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *row = z + (size_t)t * stride;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_above(row[e], e, row[best], best)) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + r] = best;
        }
        free(taken);
#ifdef ORACLE_PLANT_SHIFT_ID8
        ids[(size_t)t * k + k - 1] = (ids[(size_t)t * k + k - 1] + 1) % E; /* planted mistake */
#endif
        /* softmax over the selected logits, reference point = the top logit, summed in rank order */
        double top = (double)row[ids[(size_t)t * k]];
        double sum = 0.0;
        for (int r = 0; r < k; ++r) sum += exp((double)row[ids[(size_t)t * k + r]] - top);
        for (int r = 0; r < k; ++r)
            w[(size_t)t * k + r] = exp((double)row[ids[(size_t)t * k + r]] - top) / sum;
#ifdef ORACLE_PLANT_SWAP_W67
        if (k >= 8) { /* planted mistake: swap the weights of ranks 6 and 7, not their ids */
            double tmp = w[(size_t)t * k + 6];
            w[(size_t)t * k + 6] = w[(size_t)t * k + 7];
            w[(size_t)t * k + 7] = tmp;
        }
#endif
        if (has_gate) g[t] = 1.0 / (1.0 + exp(-(double)row[E]));
    }
    return 0;
}

/* ---------------------------------------------------------------- bucketing */
/* Stable counting sort of the n = T*k pair indices p = t*k + r by ids[p].
 * counts: [E], offsets: [E+1] (exclusive prefix sums), perm: [n]. */
int oracle_bucket(int n, int E, const int32_t *ids, int32_t *counts, int32_t *offsets,
                  int32_t *perm) {
    if (n < 0 || E <= 0) return -1;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < n; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return -1;
        counts[ids[p]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int p = 0; p < n; ++p) perm[cursor[ids[p]]++] = p;
    free(cursor);
    return 0;
}

/* ---------------------------------------------------------------- one SwiGLU FFN */
/* o[H] = Wd (silu(Wg x) * (Wu x)); gate_up is [2*I][H] with the gate rows first, down is [H][I].
 * Quantized weights take their scales as weight_at states: gu_scale covers the 2I gate and up
 * rows, dn_scale the H down rows (NULL without scales). */
static void swiglu_ffn(int H, int I, int dtype, const double *x, const void *gate_up,
                       const void *down, const void *gu_scale, const void *dn_scale,
                       double *hbuf, double *o) {
    for (int i = 0; i < I; ++i) {
        double a = 0.0, u = 0.0;
#ifdef ORACLE_PLANT_UP_SCALE_ROW
        const int su = i; /* planted mistake: the up row takes its gate row's scales */
#else
        const int su = I + i;
#endif
        for (int h = 0; h < H; ++h) {
            a += weight_at(gate_up, gu_scale, dtype, i, h, H, i) * x[h];
            u += weight_at(gate_up, gu_scale, dtype, I + i, h, H, su) * x[h];
        }
#ifdef ORACLE_PLANT_SWAP_GATE_UP
        { double tmp = a; a = u; u = tmp; } /* planted mistake: gate and up rows exchanged */
#endif
        hbuf[i] = a / (1.0 + exp(-a)) * u;
    }
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += weight_at(down, dn_scale, dtype, h, i, I, h) * hbuf[i];
        o[h] = acc;
    }
}

/* ---------------------------------------------------------------- the layer output */
/* For each token t = tokens[j] (j < n_tok): y[j][:] = sum_r w[t][r] * FFN_{ids[t][r]}(x_t)
 * + g[t] * FFN_shared(x_t). gate_up is [E][2I][H], down is [E][H][I]; the shared expert is
 * skipped when Is == 0. ids/w hold k entries per token; g may be NULL iff Is == 0. x has element
 * type xdtype, the expert weights wdtype. With wdtype FP8 the four scale arrays (fp32) give each
 * weight row's scale: gu_scale [E][2I], dn_scale [E][H], sgu_scale [2Is], sdn_scale [H]; with
 * MXFP4 the matrices hold packed codes ([E][2I][H/2], [E][H][I/2], [2Is][H/2], [H][Is/2] bytes)
 * and the scale arrays E8M0 bytes, one per 32 weights of a row: [E][2I][H/32], [E][H][I/32],
 * [2Is][H/32], [H][Is/32]. */
int oracle_forward_w(int n_tok, const int32_t *tokens, int T, int H, int E, int I, int Is, int k,
                     int xdtype, int wdtype, const void *x, const void *gate_up, const void *down,
                     const void *shared_gate_up, const void *shared_down, const void *gu_scale,
                     const void *dn_scale, const void *sgu_scale, const void *sdn_scale,
                     const int32_t *ids, const double *w, const double *g, double *y) {
    if (n_tok < 0 || H <= 0 || E <= 0 || I <= 0 || Is < 0 || k <= 0) return -1;
    if (xdtype != ORACLE_F32 && xdtype != ORACLE_BF16) return -1;
    if (wdtype < ORACLE_F32 || wdtype > ORACLE_MXFP4) return -1;
    if (Is > 0 && (!shared_gate_up || !shared_down || !g)) return -1;
    const int scaled = wdtype == ORACLE_FP8 || wdtype == ORACLE_MXFP4;
    if (scaled && (!gu_scale || !dn_scale || (Is > 0 && (!sgu_scale || !sdn_scale)))) return -1;
    if (wdtype == ORACLE_MXFP4 && (H % MX_BLOCK || I % MX_BLOCK || Is % MX_BLOCK)) return -1;
    for (int j = 0; j < n_tok; ++j)
        if (tokens[j] < 0 || tokens[j] >= T) return -1;
    const size_t gu_b = matrix_bytes(wdtype, 2 * I, H), dn_b = matrix_bytes(wdtype, H, I);
    const size_t gus_b = scale_bytes(wdtype, 2 * I, H), dns_b = scale_bytes(wdtype, H, I);
    const int Imax = I > Is ? I : Is;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int j = 0; j < n_tok; ++j) {
        const int t = tokens[j];
        double *xt = (double *)malloc(sizeof(double) * (size_t)H);
        double *hb = (double *)malloc(sizeof(double) * (size_t)Imax);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        double *yj = y + (size_t)j * H;
        for (int h = 0; h < H; ++h) xt[h] = load_elem(x, xdtype, (size_t)t * H + h);
        for (int h = 0; h < H; ++h) yj[h] = 0.0;
        for (int r = 0; r < k; ++r) {
            const int e = ids[(size_t)t * k + r];
            if (e < 0 || e >= E) { bad = 1; break; }
            const char *gu = (const char *)gate_up + (size_t)e * gu_b;
            const char *dn = (const char *)down + (size_t)e * dn_b;
            swiglu_ffn(H, I, wdtype, xt, gu, dn,
                       scaled ? (const char *)gu_scale + (size_t)e * gus_b : NULL,
                       scaled ? (const char *)dn_scale + (size_t)e * dns_b : NULL, hb, o);
            const double wk = w[(size_t)t * k + r];
            for (int h = 0; h < H; ++h) yj[h] += wk * o[h];
        }
        if (Is > 0) {
            swiglu_ffn(H, Is, wdtype, xt, shared_gate_up, shared_down, scaled ? sgu_scale : NULL,
                       scaled ? sdn_scale : NULL, hb, o);
            for (int h = 0; h < H; ++h) yj[h] += g[t] * o[h];
        }
        free(xt);
        free(hb);
        free(o);
    }
    return bad ? -1 : 0;
}

/* The same with one element type for x and the weights (no scales). */
int oracle_forward(int n_tok, const int32_t *tokens, int T, int H, int E, int I, int Is, int k,
                   int dtype, const void *x, const void *gate_up, const void *down,
                   const void *shared_gate_up, const void *shared_down, const int32_t *ids,
                   const double *w, const double *g, double *y) {
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    return oracle_forward_w(n_tok, tokens, T, H, E, I, Is, k, dtype, dtype, x, gate_up, down,
                            shared_gate_up, shared_down, NULL, NULL, NULL, NULL, ids, w, g, y);
}

/* Number of OpenMP threads a parallel region of this library uses (for reporting). */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Thread count of the parallel regions that follow (n > 0); the host baseline times the oracle
 * on one thread and on every thread the process may use. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
