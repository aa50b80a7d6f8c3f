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

/* Widen one stored element to double. bf16 is the top half of an fp32 word, so the value is the
 * 16 stored bits shifted into the high half; the conversion is exact. */
static double load_elem(const void *base, int dtype, size_t i) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
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
static void swiglu_ffn(int H, int I, int dtype, const double *x, const void *gate_up,
                       const void *down, double *hbuf, double *o) {
    for (int i = 0; i < I; ++i) {
        double a = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            a += load_elem(gate_up, dtype, (size_t)i * H + h) * x[h];
            u += load_elem(gate_up, dtype, (size_t)(I + i) * H + h) * x[h];
        }
#ifdef ORACLE_PLANT_SWAP_GATE_UP
        { double tmp = a; a = u; u = tmp; } /* planted mistake: gate and up rows exchanged */
#endif
        hbuf[i] = a / (1.0 + exp(-a)) * u;
    }
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += load_elem(down, dtype, (size_t)h * I + i) * hbuf[i];
        o[h] = acc;
    }
}

/* ---------------------------------------------------------------- the layer output */
/* For each token t = tokens[j] (j < n_tok): y[j][:] = sum_r w[t][r] * FFN_{ids[t][r]}(x_t)
 * + g[t] * FFN_shared(x_t). gate_up is [E][2I][H], down is [E][H][I]; the shared expert is
 * skipped when Is == 0. ids/w hold k entries per token; g may be NULL iff Is == 0. */
int oracle_forward(int n_tok, const int32_t *tokens, int T, int H, int E, int I, int Is, int k,
                   int dtype, const void *x, const void *gate_up, const void *down,
                   const void *shared_gate_up, const void *shared_down, const int32_t *ids,
                   const double *w, const double *g, double *y) {
    if (n_tok < 0 || H <= 0 || E <= 0 || I <= 0 || Is < 0 || k <= 0) return -1;
    if (Is > 0 && (!shared_gate_up || !shared_down || !g)) return -1;
    for (int j = 0; j < n_tok; ++j)
        if (tokens[j] < 0 || tokens[j] >= T) return -1;
    const size_t esz = dtype == ORACLE_F32 ? 4 : 2;
    const int Imax = I > Is ? I : Is;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int j = 0; j < n_tok; ++j) {
        const int t = tokens[j];
        double *xt = (double *)malloc(sizeof(double) * (size_t)H);
        double *hb = (double *)malloc(sizeof(double) * (size_t)Imax);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        double *yj = y + (size_t)j * H;
        for (int h = 0; h < H; ++h) xt[h] = load_elem(x, dtype, (size_t)t * H + h);
        for (int h = 0; h < H; ++h) yj[h] = 0.0;
        for (int r = 0; r < k; ++r) {
            const int e = ids[(size_t)t * k + r];
            if (e < 0 || e >= E) { bad = 1; break; }
            const char *gu = (const char *)gate_up + (size_t)e * 2 * I * H * esz;
            const char *dn = (const char *)down + (size_t)e * H * I * esz;
            swiglu_ffn(H, I, dtype, xt, gu, dn, hb, o);
            const double wk = w[(size_t)t * k + r];
            for (int h = 0; h < H; ++h) yj[h] += wk * o[h];
        }
        if (Is > 0) {
            swiglu_ffn(H, Is, dtype, xt, shared_gate_up, shared_down, hb, o);
            for (int h = 0; h < H; ++h) yj[h] += g[t] * o[h];
        }
        free(xt);
        free(hb);
        free(o);
    }
    return bad ? -1 : 0;
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
