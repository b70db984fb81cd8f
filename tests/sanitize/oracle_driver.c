/*
 * oracle_driver.c -- the fp64 oracle (oracle/gdn_oracle.c) on small edge-case
 * problems, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py: empty and one-token sequences, conv states, a
 * value-head range, every io dtype, no conv / no gate, the conv step alone,
 * and rejected arguments.  Every buffer is allocated at its exact size, so an
 * access past any of them stops the run.  Prints "ALL OK" and exits 0 when
 * every case returns what it should and every output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/gdn_oracle.h"

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* uniform in (-1, 1) from a 64-bit LCG */
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return ((double)(rng >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}

/* element size of an oracle dtype */
static size_t esize(int dt) { return dt == GDN_ORACLE_F32 ? 4 : dt == GDN_ORACLE_BF16 ? 2 : 8; }

/* n random values of dtype dt scaled by s; bf16 as the upper half of an fp32 */
static void* rand_buf(size_t n, int dt, double s) {
    void* p = malloc(n ? n * esize(dt) : 1);
    for (size_t i = 0; i < n; ++i) {
        const double x = s * urand();
        if (dt == GDN_ORACLE_F32) ((float*)p)[i] = (float)x;
        else if (dt == GDN_ORACLE_F64) ((double*)p)[i] = x;
        else {
            float f = (float)x;
            uint32_t u;
            memcpy(&u, &f, 4);
            ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
        }
    }
    return p;
}

static int all_finite(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

typedef struct {
    int N, Hk, Hv, d, K, io, gate_dt, state_dt, h0, h1;
    const int32_t* lens;
    int conv, gated, states;
} Case;

static void run_case(const Case* c) {
    int32_t* cu = malloc(sizeof(int32_t) * (c->N + 1));
    cu[0] = 0;
    for (int n = 0; n < c->N; ++n) cu[n + 1] = cu[n] + c->lens[n];
    const int64_t T = cu[c->N];
    const int d = c->d, Cch = 2 * c->Hk * d + c->Hv * d, nh = c->h1 - c->h0;
    gdn_oracle_desc D = {c->N, T, c->Hk, c->Hv, d, d, c->K, c->io, c->gate_dt, c->state_dt, 1,
                         1.0, 1e-6, 1e-6, c->h0, c->h1, 2};
    void* q = rand_buf((size_t)T * c->Hk * d, c->io, 1.0);
    void* k = rand_buf((size_t)T * c->Hk * d, c->io, 1.0);
    void* v = rand_buf((size_t)T * c->Hv * d, c->io, 1.0);
    void* z = c->gated ? rand_buf((size_t)T * c->Hv * d, c->io, 1.0) : NULL;
    void* nw = c->gated ? rand_buf((size_t)d, c->io, 1.0) : NULL;
    void* cw = c->conv ? rand_buf((size_t)Cch * c->K, c->io, 0.5) : NULL;
    void* g = rand_buf((size_t)T * c->Hv, c->gate_dt, 1.0);
    void* beta = rand_buf((size_t)T * c->Hv, c->gate_dt, 1.0);
    /* g <= 0 (log-decay), beta in [0, 1] */
    for (int64_t i = 0; i < T * c->Hv; ++i) {
        if (c->gate_dt == GDN_ORACLE_F32) {
            ((float*)g)[i] = -fabsf(((float*)g)[i]);
            ((float*)beta)[i] = fabsf(((float*)beta)[i]);
        } else {
            ((double*)g)[i] = -fabs(((double*)g)[i]);
            ((double*)beta)[i] = fabs(((double*)beta)[i]);
        }
    }
    void* s0 = c->states ? rand_buf((size_t)c->N * c->Hv * d * d, c->state_dt, 0.01) : NULL;
    void* cs0 = (c->states && c->conv) ? rand_buf((size_t)c->N * (c->K - 1) * Cch, c->io, 0.01) : NULL;
    double* out = malloc(sizeof(double) * ((size_t)T * nh * d + 1));
    double* fs = malloc(sizeof(double) * (size_t)c->N * nh * d * d);
    void* cso = c->conv ? malloc(esize(c->io) * (size_t)c->N * (c->K - 1) * Cch) : NULL;

    const int rc = gdn_oracle_prefill(&D, q, k, v, g, beta, z, cw, nw, cu, s0, cs0, out, fs, cso);
    CHECK(rc == 0);
    CHECK(all_finite(out, (size_t)T * nh * d));
    CHECK(all_finite(fs, (size_t)c->N * nh * d * d));
    /* a zero-length sequence passes its states through */
    for (int n = 0; n < c->N; ++n) {
        if (c->lens[n] != 0) continue;
        for (int j = 0; j < nh && c->state_dt == GDN_ORACLE_F64 && s0; ++j)
            CHECK(memcmp(fs + ((size_t)n * nh + j) * d * d,
                         (const double*)s0 + ((size_t)n * c->Hv + c->h0 + j) * d * d,
                         sizeof(double) * d * d) == 0);
        if (cso && cs0)
            CHECK(memcmp((char*)cso + esize(c->io) * (size_t)n * (c->K - 1) * Cch,
                         (char*)cs0 + esize(c->io) * (size_t)n * (c->K - 1) * Cch,
                         esize(c->io) * (size_t)(c->K - 1) * Cch) == 0);
    }
    if (c->conv) {
        double* y = malloc(sizeof(double) * ((size_t)T * Cch + 1));
        CHECK(gdn_oracle_conv_silu(&D, q, k, v, cw, cu, cs0, y) == 0);
        CHECK(all_finite(y, (size_t)T * Cch));
        free(y);
    }
    free(cu); free(q); free(k); free(v); free(z); free(nw); free(cw); free(g); free(beta);
    free(s0); free(cs0); free(out); free(fs); free(cso);
}

static void rejected(void) {
    int32_t cu[3] = {0, 2, 5};
    double out[5 * 2 * 4], fs[2 * 2 * 16];
    float x[5 * 2 * 4], gb[5 * 2];
    memset(x, 0, sizeof(x));
    memset(gb, 0, sizeof(gb));
    const gdn_oracle_desc ok = {2, 5, 1, 2, 4, 4, 4, GDN_ORACLE_F32, GDN_ORACLE_F32, GDN_ORACLE_F32,
                                1, 1.0, 1e-6, 1e-6, 0, 2, 1};
    CHECK(gdn_oracle_prefill(&ok, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == 0);
    gdn_oracle_desc d = ok;
    d.num_seqs = 0;
    CHECK(gdn_oracle_prefill(&d, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
    d = ok;
    d.num_k_heads = 3;
    CHECK(gdn_oracle_prefill(&d, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
    d = ok;
    d.total_tokens = 4;   /* != cu[N] */
    CHECK(gdn_oracle_prefill(&d, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
    d = ok;
    d.head_end = 3;
    CHECK(gdn_oracle_prefill(&d, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
    d = ok;
    d.head_begin = 2;
    d.head_end = 1;
    CHECK(gdn_oracle_prefill(&d, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
    int32_t bad_cu[3] = {0, 3, 2};   /* decreasing, cu[N] = 2 */
    d = ok;
    d.total_tokens = 2;
    CHECK(gdn_oracle_prefill(&d, x, x, x, gb, gb, NULL, NULL, NULL, bad_cu, NULL, NULL, out, fs, NULL) == -1);
    CHECK(gdn_oracle_prefill(&ok, NULL, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
    CHECK(gdn_oracle_prefill(&ok, x, x, x, gb, gb, NULL, NULL, NULL, NULL, NULL, NULL, out, fs, NULL) == -1);
    CHECK(gdn_oracle_prefill(NULL, x, x, x, gb, gb, NULL, NULL, NULL, cu, NULL, NULL, out, fs, NULL) == -1);
}

int main(void) {
    static const int32_t lens_a[] = {0, 1, 5, 70};
    static const int32_t lens_b[] = {3};
    static const int32_t lens_c[] = {2, 0, 0, 9};
    const Case cases[] = {
        /* N  Hk Hv  d  K  io                gate             state            h0 h1 lens  conv gated states */
        {4, 1, 2, 8, 4, GDN_ORACLE_F32, GDN_ORACLE_F32, GDN_ORACLE_F32, 0, 2, lens_a, 1, 1, 1},
        {4, 1, 2, 8, 4, GDN_ORACLE_BF16, GDN_ORACLE_F32, GDN_ORACLE_BF16, 1, 2, lens_a, 1, 1, 1},
        {4, 2, 4, 4, 4, GDN_ORACLE_F64, GDN_ORACLE_F64, GDN_ORACLE_F64, 1, 3, lens_c, 1, 1, 1},
        {1, 1, 1, 16, 4, GDN_ORACLE_F32, GDN_ORACLE_F32, GDN_ORACLE_F32, 0, 1, lens_b, 0, 0, 0},
        {4, 1, 3, 8, 2, GDN_ORACLE_BF16, GDN_ORACLE_F32, GDN_ORACLE_F32, 0, 3, lens_c, 1, 0, 1},
        {1, 1, 2, 8, 4, GDN_ORACLE_F32, GDN_ORACLE_F64, GDN_ORACLE_F64, 0, 2, lens_b, 1, 1, 1},
    };
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) run_case(&cases[i]);
    rejected();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ALL OK\n");
    return 0;
}
