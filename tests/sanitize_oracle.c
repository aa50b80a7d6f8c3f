/* Drives every entry point of the oracle (oracle/moe_oracle.c, compiled into this program) on
 * small random layers in the three weight formats, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle.py). Exits non-zero on any failed call; the
 * sanitizers abort on any invalid access. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_logits(int, int, int, int, const void *, const void *, const float *, float *);
int oracle_select(int, int, int, const float *, int, int, int32_t *, double *, double *);
int oracle_bucket(int, int, const int32_t *, int32_t *, int32_t *, int32_t *);
int oracle_forward_w(int, const int32_t *, int, int, int, int, int, int, int, int, const void *,
                     const void *, const void *, const void *, const void *, const void *,
                     const void *, const void *, const void *, const int32_t *, const double *,
                     const double *, double *);
double oracle_e4m3_value(uint8_t);
double oracle_e2m1_value(uint8_t);
double oracle_e8m0_value(uint8_t);

static uint64_t rng = 88172645463325252ull;
static uint32_t next32(void) { /* xorshift64 */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (uint32_t)(rng >> 32);
}
static uint16_t bf16_of(float v) { /* round to nearest even */
    uint32_t u; memcpy(&u, &v, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float unif(void) { return (float)next32() / 4294967296.0f * 2.0f - 1.0f; }
static void *fill_bf16(size_t n, float s) {
    uint16_t *p = malloc(n * 2);
    for (size_t i = 0; i < n; ++i) p[i] = bf16_of(unif() * s);
    return p;
}
static void *fill_bytes(size_t n, int lo, int hi) {
    uint8_t *p = malloc(n);
    for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(lo + (int)(next32() % (uint32_t)(hi - lo + 1)));
    return p;
}

int main(void) {
    enum { T = 5, H = 64, E = 16, I = 32, Is = 32, K = 8, R = E + 1 };
    void *x = fill_bf16((size_t)T * H, 1.0f), *wr = fill_bf16((size_t)R * H, 0.125f);
    float bias[R];
    for (int r = 0; r < R; ++r) bias[r] = unif();
    float *z = malloc(sizeof(float) * T * R);
    int32_t ids[T * K], counts[E], offsets[E + 1], perm[T * K], tokens[T];
    double w[T * K], g[T], *y = malloc(sizeof(double) * T * H);
    if (oracle_logits(T, H, R, 1, x, wr, bias, z)) return 1;
    if (oracle_select(T, E, R, z, 1, K, ids, w, g)) return 2;
    if (oracle_bucket(T * K, E, ids, counts, offsets, perm)) return 3;
    for (int t = 0; t < T; ++t) tokens[t] = T - 1 - t;
    double sum = 0.0;
    for (int fmt = 1; fmt <= 3; ++fmt) { /* bf16, FP8 E4M3, MXFP4 */
        const size_t gu_n = (size_t)E * 2 * I * H, dn_n = (size_t)E * H * I;
        const size_t sgu_n = (size_t)2 * Is * H, sdn_n = (size_t)H * Is;
        void *gu, *dn, *sgu, *sdn, *gus = NULL, *dns = NULL, *sgus = NULL, *sdns = NULL;
        if (fmt == 1) {
            gu = fill_bf16(gu_n, 0.125f); dn = fill_bf16(dn_n, 0.18f);
            sgu = fill_bf16(sgu_n, 0.125f); sdn = fill_bf16(sdn_n, 0.18f);
        } else if (fmt == 2) {
            gu = fill_bytes(gu_n, 0, 0x7E); dn = fill_bytes(dn_n, 0x80, 0xFE);
            sgu = fill_bytes(sgu_n, 0, 0x7E); sdn = fill_bytes(sdn_n, 0, 0x7E);
            float *a = malloc(sizeof(float) * E * 2 * I), *b = malloc(sizeof(float) * E * H);
            float *c = malloc(sizeof(float) * 2 * Is), *d = malloc(sizeof(float) * H);
            for (int i = 0; i < E * 2 * I; ++i) a[i] = ldexpf(1.0f, -8);
            for (int i = 0; i < E * H; ++i) b[i] = ldexpf(1.0f, -9);
            for (int i = 0; i < 2 * Is; ++i) c[i] = ldexpf(1.0f, -8);
            for (int i = 0; i < H; ++i) d[i] = ldexpf(1.0f, -9);
            gus = a; dns = b; sgus = c; sdns = d;
        } else {
            gu = fill_bytes(gu_n / 2, 0, 255); dn = fill_bytes(dn_n / 2, 0, 255);
            sgu = fill_bytes(sgu_n / 2, 0, 255); sdn = fill_bytes(sdn_n / 2, 0, 255);
            gus = fill_bytes(gu_n / 32, 118, 124); dns = fill_bytes(dn_n / 32, 118, 124);
            sgus = fill_bytes(sgu_n / 32, 118, 124); sdns = fill_bytes(sdn_n / 32, 118, 124);
        }
        if (oracle_forward_w(T, tokens, T, H, E, I, Is, K, 1, fmt, x, gu, dn, sgu, sdn, gus, dns,
                             sgus, sdns, ids, w, g, y)) return 10 + fmt;
        for (int i = 0; i < T * H; ++i) sum += y[i];
        free(gu); free(dn); free(sgu); free(sdn); free(gus); free(dns); free(sgus); free(sdns);
    }
    for (int c = 0; c < 256; ++c)
        sum += oracle_e2m1_value((uint8_t)(c & 15)) + (c == 255 ? 0.0 : oracle_e8m0_value((uint8_t)c) * 1e-40) +
               ((c & 0x7F) == 0x7F ? 0.0 : oracle_e4m3_value((uint8_t)c));
    free(x); free(wr); free(z); free(y);
    printf("checksum %.17g\n", sum);
    return isfinite(sum) ? 0 : 20;
}
