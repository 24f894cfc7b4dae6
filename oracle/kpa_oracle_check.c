/*
 * Driver for a sanitizer build of the streaming C oracle (kpa_oracle.c).
 *
 * TEST INFRASTRUCTURE ONLY.  Built twice by the CPU test-suite -- once with
 * AddressSanitizer and UndefinedBehaviorSanitizer, once plainly -- and run
 * over a fixed set of shapes: non-degenerate and degenerate splits, unequal
 * ranks, ragged and empty contexts, causal and non-causal multi-query
 * decode, float32 and bfloat16 inputs, all rows and a selection of rows.
 * It prints every output and log-sum-exp value; the two builds must print
 * the same text and the sanitized one must report nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kpa_oracle_decode(int p1, int p2, int q1, int q2, int rk, int rv, double base,
                      int batch, int stride_s, int elem_kind,
                      const void* ak, const void* bk, const void* av, const void* bv,
                      const int32_t* positions, const int32_t* ctx_len,
                      int n_q, int causal, const float* q, const int32_t* q_pos,
                      const int32_t* items, int n_items,
                      double* out, double* lse, int n_threads);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* uniform in [-1, 1) from a 64-bit linear congruential generator */
static float next_uniform(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

/* n factor values in the requested encoding (0 float32, 1 bfloat16 bits) */
static void* make_factors(size_t n, int kind) {
    if (kind == 0) {
        float* f = (float*)malloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) f[i] = next_uniform();
        return f;
    }
    uint16_t* h = (uint16_t*)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        float v = next_uniform();
        uint32_t u;
        memcpy(&u, &v, sizeof u);
        h[i] = (uint16_t)(u >> 16);
    }
    return h;
}

typedef struct {
    int p1, p2, q1, q2, rk, rv, batch, slots, n_q, causal, kind, use_items;
} shape;

static int run_case(const shape* c) {
    const int h = c->p1 * c->p2, d_h = c->q1 * c->q2;
    const size_t tok = (size_t)c->batch * c->slots;
    void* ak = make_factors(tok * c->rk * c->p1 * c->q1, c->kind);
    void* bk = make_factors(tok * c->rk * c->p2 * c->q2, c->kind);
    void* av = make_factors(tok * c->rv * c->p1 * c->q1, c->kind);
    void* bv = make_factors(tok * c->rv * c->p2 * c->q2, c->kind);
    int32_t* pos = (int32_t*)malloc(tok * sizeof(int32_t));
    for (size_t t = 0; t < tok; ++t) pos[t] = (int32_t)(t % c->slots) * 37;
    int32_t* ctx = (int32_t*)malloc(c->batch * sizeof(int32_t));
    for (int b = 0; b < c->batch; ++b) ctx[b] = (b == 1) ? 0 : c->slots - (b % 3);  /* ragged, one empty */
    const size_t nq_rows = (size_t)c->batch * c->n_q;
    float* q = (float*)malloc(nq_rows * h * d_h * sizeof(float));
    for (size_t i = 0; i < nq_rows * h * d_h; ++i) q[i] = 2.0f * next_uniform();
    int32_t* qp = (int32_t*)malloc(nq_rows * sizeof(int32_t));
    for (size_t i = 0; i < nq_rows; ++i) qp[i] = (int32_t)(i * 101 % 5000);
    int n_items = c->batch * c->n_q * h;
    int32_t* items = NULL;
    if (c->use_items) {
        n_items = 5;
        items = (int32_t*)malloc(3 * n_items * sizeof(int32_t));
        for (int k = 0; k < n_items; ++k) {
            items[3 * k] = (k * 7) % c->batch;
            items[3 * k + 1] = (k * 3) % c->n_q;
            items[3 * k + 2] = (k * 5) % h;
        }
    }
    double* out = (double*)malloc((size_t)n_items * d_h * sizeof(double));
    double* lse = (double*)malloc((size_t)n_items * sizeof(double));
    int rc = kpa_oracle_decode(c->p1, c->p2, c->q1, c->q2, c->rk, c->rv, 10000.0, c->batch, c->slots, c->kind,
                               ak, bk, av, bv, pos, ctx, c->n_q, c->causal, q, qp, items, n_items, out, lse, 0);
    if (rc == 0) {
        for (int k = 0; k < n_items; ++k) {
            printf("lse %.17g\n", lse[k]);
            for (int j = 0; j < d_h; ++j) printf("%.17g\n", out[(size_t)k * d_h + j]);
        }
    }
    free(ak); free(bk); free(av); free(bv); free(pos); free(ctx); free(q); free(qp); free(items);
    free(out); free(lse);
    return rc;
}

int main(void) {
    static const shape cases[] = {
        /* p1 p2 q1 q2 rk rv batch slots n_q causal kind items */
        {2, 2, 4, 4, 2, 2, 3, 11, 1, 1, 0, 0},
        {4, 4, 8, 16, 2, 2, 2, 9, 1, 1, 1, 0},
        {12, 1, 1, 64, 2, 2, 3, 7, 1, 1, 1, 1},
        {3, 2, 1, 6, 1, 3, 4, 13, 3, 1, 0, 0},
        {2, 3, 3, 2, 3, 1, 3, 6, 2, 0, 1, 0},
        {4, 8, 16, 8, 4, 4, 2, 20, 4, 1, 1, 1},
        {1, 1, 2, 2, 1, 1, 2, 1, 1, 1, 0, 0},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
        printf("case %zu\n", i);
        if (run_case(&cases[i]) != 0) {
            fprintf(stderr, "case %zu failed\n", i);
            return 1;
        }
    }
    /* invalid arguments are refused */
    if (kpa_oracle_decode(2, 2, 4, 3, 1, 1, 10000.0, 1, 1, 0, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, NULL,
                          NULL, NULL, 0, NULL, NULL, 0) != -1) {
        fprintf(stderr, "odd d2 accepted\n");
        return 1;
    }
    return 0;
}
