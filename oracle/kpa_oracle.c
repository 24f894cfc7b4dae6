/*
 * Streaming float64 oracle for KPA factor-cache decode (plain C + OpenMP).
 *
 * TEST INFRASTRUCTURE ONLY: used by the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark.  It shares no code with the HIP library.
 *
 * It computes exactly the definition that oracle/kpa_ref.py writes out with
 * NumPy, streamed one cached token at a time so that full K/V of a long
 * context are never held in memory:
 *   for every visible slot s of a (sequence, query, head) item
 *     k = (1/R_K) sum_r (A^K_r)_{i1} (x) (B^K_r)_{i2}         [KPA] Eq. (3)
 *     k' = R_KPA(pos_s) k, R_KPA = I_{d1} (x) R^(2)(pos_s)     [KPA] Def. 2.3
 *     z_s = q' . k' / sqrt(d_h), q' = R_KPA(q_pos) q           [KPA] §2.3
 *   m = max_s z_s, l = sum_s exp(z_s - m)
 *   o = sum_s exp(z_s - m) v_s / l,  v = (1/R_V) sum_r (A^V_r)_{i1} (x) (B^V_r)_{i2}
 *   lse = m + log l
 * R_KPA is applied as the 2x2 rotations of consecutive feature pairs inside
 * each d2 block (the same operator as the explicit matrix; [KPA] Def. 2.3),
 * theta_m = base^(-2m/d2).
 *
 * Sources: [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression
 * via Structured Factorization" (arXiv 2610.12657).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Input element encodings (how the caller's arrays are stored, not how they
 * are computed with): 0 = float32, 1 = bfloat16 bit patterns (uint16). */
static double load_elem(const void* base, size_t idx, int kind) {
    if (kind == 0) return (double)((const float*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    int p1, p2, q1, q2, rk, rv;
    double base;
    int batch, stride_s; /* token-dimension stride of the factor arrays */
    int elem_kind;
    const void *ak, *bk, *av, *bv;
    const int32_t* positions; /* [batch][stride_s] */
    const int32_t* ctx_len;   /* [batch] */
    int n_q, causal;
    const float* q;           /* [batch][n_q][h][d_h] */
    const int32_t* q_pos;     /* [batch][n_q] */
} problem;

/* Rotate the d_h-vector x in place by R_KPA(pos): pairs (2m, 2m+1) inside
 * every d2 block turn by angle pos * theta_m. */
static void rotate_kpa(double* x, int q1, int q2, double pos, double base) {
    for (int m = 0; m < q2 / 2; ++m) {
        double theta = pow(base, -2.0 * (double)m / (double)q2);
        double ang = pos * theta;
        double c = cos(ang), s = sin(ang);
        for (int j1 = 0; j1 < q1; ++j1) {
            double* e = x + (size_t)j1 * q2 + 2 * m;
            double x0 = e[0], x1 = e[1];
            e[0] = x0 * c - x1 * s;
            e[1] = x0 * s + x1 * c;
        }
    }
}

/* One head row of (1/R) sum_r A_r (x) B_r for slot s of sequence b. */
static void kron_row(const problem* P, const void* a, const void* bfac, int r_n,
                     int b, int s, int i1, int i2, double* row) {
    const int p1 = P->p1, p2 = P->p2, q1 = P->q1, q2 = P->q2;
    const int d_h = q1 * q2;
    for (int j = 0; j < d_h; ++j) row[j] = 0.0;
    size_t tok = (size_t)b * P->stride_s + (size_t)s;
    for (int r = 0; r < r_n; ++r) {
        size_t abase = ((tok * r_n + r) * p1 + i1) * (size_t)q1;
        size_t bbase = ((tok * r_n + r) * p2 + i2) * (size_t)q2;
        for (int j1 = 0; j1 < q1; ++j1) {
            double av = load_elem(a, abase + j1, P->elem_kind);
            for (int j2 = 0; j2 < q2; ++j2)
                row[j1 * q2 + j2] += av * load_elem(bfac, bbase + j2, P->elem_kind);
        }
    }
    for (int j = 0; j < d_h; ++j) row[j] /= (double)r_n;
}

static void one_item(const problem* P, int b, int n, int head, double* out, double* lse_out,
                     double* z, double* krow, double* qrot) {
    const int p2 = P->p2, q1 = P->q1, q2 = P->q2;
    const int h = P->p1 * p2, d_h = q1 * q2;
    const int i1 = head / p2, i2 = head % p2;
    int ctx = P->ctx_len[b];
    if (ctx > P->stride_s) ctx = P->stride_s;
    if (ctx < 0) ctx = 0;
    int visible = P->causal ? ctx - P->n_q + n + 1 : ctx;
    if (visible > ctx) visible = ctx;
    if (visible < 0) visible = 0;

    const float* qv = P->q + (((size_t)b * P->n_q + n) * h + head) * (size_t)d_h;
    for (int j = 0; j < d_h; ++j) qrot[j] = (double)qv[j];
    rotate_kpa(qrot, q1, q2, (double)P->q_pos[(size_t)b * P->n_q + n], P->base);

    const double inv_sqrt = 1.0 / sqrt((double)d_h);
    double m = -INFINITY;
    for (int s = 0; s < visible; ++s) {
        kron_row(P, P->ak, P->bk, P->rk, b, s, i1, i2, krow);
        rotate_kpa(krow, q1, q2, (double)P->positions[(size_t)b * P->stride_s + s], P->base);
        double dot = 0.0;
        for (int j = 0; j < d_h; ++j) dot += qrot[j] * krow[j];
        z[s] = dot * inv_sqrt;
        if (z[s] > m) m = z[s];
    }
    for (int j = 0; j < d_h; ++j) out[j] = 0.0;
    if (visible == 0) {
        *lse_out = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int s = 0; s < visible; ++s) {
        double w = exp(z[s] - m);
        l += w;
        kron_row(P, P->av, P->bv, P->rv, b, s, i1, i2, krow);
        for (int j = 0; j < d_h; ++j) out[j] += w * krow[j];
    }
    for (int j = 0; j < d_h; ++j) out[j] /= l;
    *lse_out = m + log(l);
}

/*
 * Compute n_items outputs.  items[k] = (b, n, head) selects one output row;
 * items == NULL means every (b, n, head) in order.  out: [n_items][d_h],
 * lse: [n_items].  Returns 0, or -1 on bad arguments / allocation failure.
 */
int kpa_oracle_decode(int p1, int p2, int q1, int q2, int rk, int rv, double base,
                      int batch, int stride_s, int elem_kind,
                      const void* ak, const void* bk, const void* av, const void* bv,
                      const int32_t* positions, const int32_t* ctx_len,
                      int n_q, int causal, const float* q, const int32_t* q_pos,
                      const int32_t* items, int n_items,
                      double* out, double* lse, int n_threads) {
    if (p1 <= 0 || p2 <= 0 || q1 <= 0 || q2 <= 0 || (q2 % 2) || rk <= 0 || rv <= 0) return -1;
    if (batch <= 0 || stride_s < 0 || n_q <= 0) return -1;
    problem P = {p1, p2, q1, q2, rk, rv, base, batch, stride_s, elem_kind,
                 ak, bk, av, bv, positions, ctx_len, n_q, causal, q, q_pos};
    const int h = p1 * p2, d_h = q1 * q2;
    int total = items ? n_items : batch * n_q * h;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(stride_s > 0 ? stride_s : 1));
        double* krow = (double*)malloc(sizeof(double) * (size_t)d_h);
        double* qrot = (double*)malloc(sizeof(double) * (size_t)d_h);
        int ok = (z && krow && qrot);
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int k = 0; k < total; ++k) {
            if (!ok) continue;
            int b, n, head;
            if (items) {
                b = items[3 * k];
                n = items[3 * k + 1];
                head = items[3 * k + 2];
            } else {
                b = k / (n_q * h);
                n = (k / h) % n_q;
                head = k % h;
            }
            one_item(&P, b, n, head, out + (size_t)k * d_h, lse + k, z, krow, qrot);
        }
        free(z);
        free(krow);
        free(qrot);
    }
    return failed ? -1 : 0;
}

/* Threads an OpenMP parallel region would use (reported with the CPU baseline). */
int kpa_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
