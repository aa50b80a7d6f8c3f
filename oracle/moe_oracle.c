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
 *   oracle_forward_w the same with FP8 expert weights: each weight is its E4M3 code's value times
 *                   its row's fp32 scale, taken exactly in fp64 before the products (the pages
 *                   name quantized expert formats - groupwise integers, FP8, NVFP4 - without
 *                   fixing one; per-row scales over OCP E4M3 codes are the reading here).
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

/* Widen one stored element to double. bf16 is the top half of an fp32 word, so the value is the
 * 16 stored bits shifted into the high half; the conversion is exact. An FP8 element is its
 * code's value times the fp32 scale of its row (given by the caller). */
static double load_elem(const void *base, int dtype, size_t i) {
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
/* o[H] = Wd (silu(Wg x) * (Wu x)); gate_up is [2*I][H] with the gate rows first, down is [H][I]. */
/* With scales (FP8 weights): element (row, col) of a matrix is value(code) * scale[row]; gu_scale
 * has 2I entries (gate rows, then up rows), dn_scale H. Without, the scales are 1. */
static void swiglu_ffn(int H, int I, int dtype, const double *x, const void *gate_up,
                       const void *down, const float *gu_scale, const float *dn_scale,
                       double *hbuf, double *o) {
    for (int i = 0; i < I; ++i) {
        double a = 0.0, u = 0.0;
        const double sg = gu_scale ? (double)gu_scale[i] : 1.0;
#ifdef ORACLE_PLANT_UP_SCALE_ROW
        const double su = gu_scale ? (double)gu_scale[i] : 1.0; /* planted: the gate row's scale */
#else
        const double su = gu_scale ? (double)gu_scale[I + i] : 1.0;
#endif
        for (int h = 0; h < H; ++h) {
            a += load_elem(gate_up, dtype, (size_t)i * H + h) * sg * x[h];
            u += load_elem(gate_up, dtype, (size_t)(I + i) * H + h) * su * x[h];
        }
#ifdef ORACLE_PLANT_SWAP_GATE_UP
        { double tmp = a; a = u; u = tmp; } /* planted mistake: gate and up rows exchanged */
#endif
        hbuf[i] = a / (1.0 + exp(-a)) * u;
    }
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        const double sd = dn_scale ? (double)dn_scale[h] : 1.0;
        for (int i = 0; i < I; ++i) acc += load_elem(down, dtype, (size_t)h * I + i) * sd * hbuf[i];
        o[h] = acc;
    }
}

/* ---------------------------------------------------------------- the layer output */
/* For each token t = tokens[j] (j < n_tok): y[j][:] = sum_r w[t][r] * FFN_{ids[t][r]}(x_t)
 * + g[t] * FFN_shared(x_t). gate_up is [E][2I][H], down is [E][H][I]; the shared expert is
 * skipped when Is == 0. ids/w hold k entries per token; g may be NULL iff Is == 0. x has element
 * type xdtype, the expert weights wdtype; with wdtype FP8 the four scale arrays give each weight
 * row's scale: gu_scale [E][2I], dn_scale [E][H], sgu_scale [2Is], sdn_scale [H]. */
int oracle_forward_w(int n_tok, const int32_t *tokens, int T, int H, int E, int I, int Is, int k,
                     int xdtype, int wdtype, const void *x, const void *gate_up, const void *down,
                     const void *shared_gate_up, const void *shared_down, const float *gu_scale,
                     const float *dn_scale, const float *sgu_scale, const float *sdn_scale,
                     const int32_t *ids, const double *w, const double *g, double *y) {
    if (n_tok < 0 || H <= 0 || E <= 0 || I <= 0 || Is < 0 || k <= 0) return -1;
    if (xdtype != ORACLE_F32 && xdtype != ORACLE_BF16) return -1;
    if (Is > 0 && (!shared_gate_up || !shared_down || !g)) return -1;
    const int scaled = wdtype == ORACLE_FP8;
    if (scaled && (!gu_scale || !dn_scale || (Is > 0 && (!sgu_scale || !sdn_scale)))) return -1;
    for (int j = 0; j < n_tok; ++j)
        if (tokens[j] < 0 || tokens[j] >= T) return -1;
    const size_t esz = elem_size(wdtype);
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
            const char *gu = (const char *)gate_up + (size_t)e * 2 * I * H * esz;
            const char *dn = (const char *)down + (size_t)e * H * I * esz;
            swiglu_ffn(H, I, wdtype, xt, gu, dn, scaled ? gu_scale + (size_t)e * 2 * I : NULL,
                       scaled ? dn_scale + (size_t)e * H : NULL, hb, o);
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
