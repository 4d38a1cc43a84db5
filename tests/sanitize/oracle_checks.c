/*
 * Every function of the CPU oracle (oracle/oracle.c) on small inputs, built
 * with AddressSanitizer and UndefinedBehaviorSanitizer (no recovery): layout
 * round trips in both element sizes, exchange volumes, attention in every
 * dtype with and without the causal mask, grouped heads and row subsets, the
 * gradients and their sampled form (which must equal the full computation bit
 * for bit), and the bf16 rounding on special values.  Exit status 0: every
 * check held and no sanitizer report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_seq_to_head(const void *, void *, int64_t, int64_t, int64_t, int64_t, int32_t, int32_t);
int oracle_head_to_seq(const void *, void *, int64_t, int64_t, int64_t, int64_t, int32_t, int32_t);
int64_t oracle_send_bytes(int64_t, int64_t, int64_t, int64_t, int32_t, int32_t, int32_t);
int oracle_attention(const void *, const void *, const void *, int32_t, double *, int64_t, int64_t,
                     int64_t, int64_t, int64_t, int32_t, const int64_t *, int64_t, int32_t);
int oracle_attention_backward(const void *, const void *, const void *, const void *, int32_t,
                              double *, double *, double *, double *, int64_t, int64_t, int64_t,
                              int64_t, int64_t, int32_t, int32_t, int32_t);
int oracle_attention_backward_sampled(const void *, const void *, const void *, const void *, int32_t,
                                      const int64_t *, int64_t, const int64_t *, int64_t, double *,
                                      double *, double *, int64_t, int64_t, int64_t, int64_t, int64_t,
                                      int32_t, int32_t, int32_t);
int oracle_round_bf16(const double *, double *, int64_t);

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            ++failures;                                                       \
            fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c);     \
        }                                                                     \
    } while (0)

static uint64_t state = 88172645463325252ull;
static uint64_t next(void) { /* xorshift64 */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static double unit(void) { return (double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0; }

static void fill(void *p, int32_t dtype, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        const double x = unit();
        if (dtype == 0) {
            float f = (float)x;
            uint32_t u;
            memcpy(&u, &f, 4);
            uint16_t h = (uint16_t)(u >> 16);
            memcpy((char *)p + 2 * i, &h, 2);
        } else if (dtype == 1) {
            float f = (float)x;
            memcpy((char *)p + 4 * i, &f, 4);
        } else {
            memcpy((char *)p + 8 * i, &x, 8);
        }
    }
}

static void layouts(void) {
    const int64_t shapes[][5] = {{1, 8, 4, 3, 4}, {2, 12, 6, 5, 3}, {3, 6, 2, 7, 2}, {1, 5, 5, 1, 1}};
    for (int e = 2; e <= 4; e += 2)
        for (int s = 0; s < 4; ++s) {
            const int64_t B = shapes[s][0], S = shapes[s][1], H = shapes[s][2], D = shapes[s][3];
            const int32_t P = (int32_t)shapes[s][4];
            const size_t bytes = (size_t)(B * S * H * D * e);
            unsigned char *a = malloc(bytes), *b = malloc(bytes), *c = malloc(bytes);
            for (size_t i = 0; i < bytes; ++i) a[i] = (unsigned char)next();
            CHECK(oracle_seq_to_head(a, b, B, S, H, D, P, e) == 0);
            CHECK(oracle_head_to_seq(b, c, B, S, H, D, P, e) == 0);
            CHECK(memcmp(a, c, bytes) == 0);
            for (int32_t r = 0; r < P; ++r)
                CHECK(oracle_send_bytes(B, S, H, D, P, e, r) == B * (S / P) * H * D * e * (P - 1) / P);
            free(a);
            free(b);
            free(c);
        }
    CHECK(oracle_seq_to_head(NULL, NULL, 1, 7, 4, 2, 2, 2) != 0); /* S not divisible */
    CHECK(oracle_send_bytes(1, 8, 4, 2, 2, 2, 5) < 0);              /* rank out of range */
}

static void attention(void) {
    const int64_t B = 2, S = 37, Hq = 4, Hkv = 2, D = 8;
    const int64_t rows[] = {0, 1, 17, 36, 17};
    for (int32_t dt = 0; dt < 3; ++dt) {
        const int es = dt == 0 ? 2 : dt == 1 ? 4 : 8;
        void *q = malloc((size_t)(B * S * Hq * D * es)), *k = malloc((size_t)(B * S * Hkv * D * es));
        void *v = malloc((size_t)(B * S * Hkv * D * es)), *g = malloc((size_t)(B * S * Hq * D * es));
        fill(q, dt, B * S * Hq * D);
        fill(k, dt, B * S * Hkv * D);
        fill(v, dt, B * S * Hkv * D);
        fill(g, dt, B * S * Hq * D);
        double *o = malloc(sizeof(double) * (size_t)(B * S * Hq * D));
        double *os = malloc(sizeof(double) * (size_t)(B * 5 * Hq * D));
        double *dq = malloc(sizeof(double) * (size_t)(B * S * Hq * D));
        double *dk = malloc(sizeof(double) * (size_t)(B * S * Hkv * D));
        double *dv = malloc(sizeof(double) * (size_t)(B * S * Hkv * D));
        double *lse = malloc(sizeof(double) * (size_t)(B * Hq * S));
        double *sq = malloc(sizeof(double) * (size_t)(B * 5 * Hq * D));
        double *sk = malloc(sizeof(double) * (size_t)(B * 5 * Hkv * D));
        double *sv = malloc(sizeof(double) * (size_t)(B * 5 * Hkv * D));
        for (int32_t causal = 0; causal < 2; ++causal)
            for (int32_t threads = 1; threads <= 3; threads += 2) {
                CHECK(oracle_attention(q, k, v, dt, o, B, S, Hq, Hkv, D, causal, NULL, 0, threads) == 0);
                CHECK(oracle_attention(q, k, v, dt, os, B, S, Hq, Hkv, D, causal, rows, 5, threads) == 0);
                for (int64_t b = 0; b < B; ++b)
                    for (int64_t r = 0; r < 5; ++r)
                        for (int64_t c = 0; c < Hq * D; ++c)
                            CHECK(os[(b * 5 + r) * Hq * D + c] == o[(b * S + rows[r]) * Hq * D + c]);
                for (int32_t round_o = 0; round_o < 2; ++round_o) {
                    CHECK(oracle_attention_backward(q, k, v, g, dt, dq, dk, dv, lse, B, S, Hq, Hkv, D,
                                                    causal, round_o, threads) == 0);
                    CHECK(oracle_attention_backward_sampled(q, k, v, g, dt, rows, 5, rows, 5, sq, sk, sv,
                                                            B, S, Hq, Hkv, D, causal, round_o,
                                                            threads) == 0);
                    for (int64_t b = 0; b < B; ++b)
                        for (int64_t r = 0; r < 5; ++r) { /* row 17 is listed twice: its values sit in the later slot */
                            for (int64_t c = 0; c < Hq * D; ++c)
                                CHECK(sq[(b * 5 + r) * Hq * D + c] == dq[(b * S + rows[r]) * Hq * D + c] || r == 2);
                            for (int64_t c = 0; c < Hkv * D; ++c) {
                                CHECK(sk[(b * 5 + r) * Hkv * D + c] == dk[(b * S + rows[r]) * Hkv * D + c] || r == 2);
                                CHECK(sv[(b * 5 + r) * Hkv * D + c] == dv[(b * S + rows[r]) * Hkv * D + c] || r == 2);
                            }
                        }
                    for (int64_t i = 0; i < B * Hq * S; ++i) CHECK(isfinite(lse[i]));
                }
            }
        const int64_t bad_rows[] = {S};
        CHECK(oracle_attention(q, k, v, dt, os, B, S, Hq, Hkv, D, 1, bad_rows, 1, 1) != 0);
        CHECK(oracle_attention(q, k, v, dt, o, B, S, Hq, 3, D, 1, NULL, 0, 1) != 0);
        free(q); free(k); free(v); free(g); free(o); free(os);
        free(dq); free(dk); free(dv); free(lse); free(sq); free(sk); free(sv);
    }
}

static void rounding(void) {
    const double x[] = {0.0, -0.0, 1.0, 1.0 + 0x1p-8, 1.0 + 3 * 0x1p-8, 0x1p-134, 0x1p-140,
                        255.5 * 0x1p120, 1e300, -1e300, INFINITY, -INFINITY, NAN, 3.14159};
    const double want[] = {0.0, -0.0, 1.0, 1.0, 1.0 + 0x1p-6, 0.0, 0.0,
                           INFINITY, INFINITY, -INFINITY, INFINITY, -INFINITY, NAN, 3.140625};
    double y[14];
    CHECK(oracle_round_bf16(x, y, 14) == 0);
    for (int i = 0; i < 14; ++i)
        CHECK((isnan(want[i]) && isnan(y[i])) || (y[i] == want[i] && signbit(y[i]) == signbit(want[i])));
    CHECK(oracle_round_bf16(x, y, -1) != 0);
}

int main(void) {
    layouts();
    attention();
    rounding();
    printf("oracle checks: %d failures\n", failures);
    return failures ? 1 : 0;
}
