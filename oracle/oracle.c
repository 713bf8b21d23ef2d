/*
 * CPU fp64 oracle for content-routed token-sparse attention with a
 * Lightning-Indexer-style selector.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path links,
 * loads or calls this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the GPU library: its decoders, visibility rule, score,
 * selection and softmax are written out here from the pages' definitions.
 *
 * What it computes, and where each step is defined:
 *  - Decoding of stored elements to fp64 (f32 bit-cast, bf16 = high half of
 *    an f32, OCP FP8 e4m3fn: bias 7, subnormals at exponent 0, S.1111.111 is
 *    NaN and is rejected).  The FP8 index-key format is the pages' (Fine-grained
 *    indexing, §2.1 "index K full-scan byte floor" and §3.1 on quantised index
 *    keys); the OCP flavour is our reading.
 *  - Visible set of a query row: positions j < kv_len[b] and, when causal,
 *    j <= q_pos(b,i) with q_pos(b,i) = q_pos0[b] + i (Hashing and clustering,
 *    §1.1: the candidate set is intersected with the causal set j <= i and the
 *    valid-token set; padding never takes part).  Self is visible.
 *  - Indexer score r = sum_h w_h * ReLU(<q_h, k_j>), one index key per token
 *    shared by all index heads, query-dependent head weights (Fine-grained
 *    indexing, §1.1 and §3.2, the multi-head ReLU proxy score).  fp64, summed
 *    over d ascending then h ascending.
 *  - Select: the first min(k, |V|) visible positions ordered by (score desc,
 *    position asc); remaining slots are -1; emitted in ascending position
 *    (Fine-grained indexing, §2.1 eq. (4) and the causal-prefill and
 *    tie-stability paragraphs; §3.1 lexicographic (score, index) top-k).
 *  - Attention over the selected rows only: logits scale * <Q, K_j>, one
 *    softmax over the whole candidate set (row max, exp-sum), output the
 *    p-weighted sum of V_j, LSE = max + log(sum)  (Hashing and clustering,
 *    §1.1 eq. (1) and §5.1 on one shared denominator; Fine-grained indexing,
 *    §3.2 logit definition).  An empty set gives O = 0, LSE = -inf.
 *
 * Built with gcc into liboracle.so and driven through ctypes by oracle.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };

typedef struct {
    int32_t B, n_q, n_kv, Hq, Hkv, d_qk, d_v, Hidx, d_idx, k, causal;
    double scale;
    const int32_t* kv_len;      /* host [B]; NULL -> n_kv */
    const int32_t* q_pos0;      /* host [B]; NULL -> 0 */
    const int32_t* pos_of_slot; /* host [B, n_kv]; NULL -> slot j holds position j */
} or_problem;

/* A strided view: element (i0,i1,i2,d) sits at data + i0*s0 + i1*s1 + i2*s2 + d elements. */
typedef struct {
    const void* data;
    int32_t dtype;
    int64_t s0, s1, s2;
} or_view;

/* ---------------------------------------------------------------- decode */

static double e4m3_value(uint8_t c, int* bad) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) { *bad = 1; return NAN; }
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

static double dec(const or_view* v, int64_t e, int* bad) {
    switch (v->dtype) {
    case OR_F32: {
        double x = ((const float*)v->data)[e];
        if (!isfinite(x)) *bad = 1;
        return x;
    }
    case OR_BF16: {
        uint32_t u = (uint32_t)((const uint16_t*)v->data)[e] << 16;
        float f;
        memcpy(&f, &u, 4);
        if (!isfinite(f)) *bad = 1;
        return f;
    }
    case OR_E4M3:
        return e4m3_value(((const uint8_t*)v->data)[e], bad);
    default:
        *bad = 1;
        return NAN;
    }
}

double or_decode_one(int32_t dtype, uint32_t bits) {
    int bad = 0;
    or_view v = {&bits, dtype, 0, 0, 0};
    uint16_t h = (uint16_t)bits;
    uint8_t c = (uint8_t)bits;
    if (dtype == OR_BF16) v.data = &h;
    if (dtype == OR_E4M3) v.data = &c;
    double x = dec(&v, 0, &bad);
    return x;
}

/* ------------------------------------------------------------ visibility */

static int32_t kvlen_of(const or_problem* p, int b) { return p->kv_len ? p->kv_len[b] : p->n_kv; }
static int64_t qpos_of(const or_problem* p, int b, int i) { return (int64_t)(p->q_pos0 ? p->q_pos0[b] : 0) + i; }
static int32_t pos_of(const or_problem* p, int b, int j) {
    return p->pos_of_slot ? p->pos_of_slot[(int64_t)b * p->n_kv + j] : j;
}
static int row_valid(const or_problem* p, int b, int i) { return qpos_of(p, b, i) < kvlen_of(p, b); }
static int visible(const or_problem* p, int b, int i, int j) {
    if (!row_valid(p, b, i)) return 0;
    int64_t pos = pos_of(p, b, j);
    if (pos >= kvlen_of(p, b)) return 0;
    if (p->causal && pos > qpos_of(p, b, i)) return 0;
    return 1;
}

int64_t or_count_visible(const or_problem* p) {
    int64_t n = 0;
    for (int b = 0; b < p->B; ++b)
        for (int i = 0; i < p->n_q; ++i)
            for (int j = 0; j < p->n_kv; ++j) n += visible(p, b, i, j);
    return n;
}

/* ------------------------------------------------------------- threading */

typedef struct {
    void (*fn)(void* ctx, int64_t r);
    void* ctx;
    int64_t n;
    int64_t next;
    pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* a) {
    pool_t* P = (pool_t*)a;
    for (;;) {
        pthread_mutex_lock(&P->mu);
        int64_t r = P->next++;
        pthread_mutex_unlock(&P->mu);
        if (r >= P->n) break;
        P->fn(P->ctx, r);
    }
    return 0;
}

static void pool_run(void (*fn)(void*, int64_t), void* ctx, int64_t n, int nthreads) {
    pool_t P;
    P.fn = fn; P.ctx = ctx; P.n = n; P.next = 0;
    pthread_mutex_init(&P.mu, 0);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 128) nthreads = 128;
    if (nthreads == 1 || n == 1) {
        pool_worker(&P);
    } else {
        pthread_t th[128];
        for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], 0, pool_worker, &P);
        for (int t = 0; t < nthreads; ++t) pthread_join(th[t], 0);
    }
    pthread_mutex_destroy(&P.mu);
}

/* --------------------------------------------------------------- scores */

typedef struct {
    const or_problem* p;
    or_view q, k, w;
    const int32_t* rows;
    double* out;
    int bad;
} score_ctx;

static void score_row(void* c_, int64_t r) {
    score_ctx* c = (score_ctx*)c_;
    const or_problem* p = c->p;
    int row = c->rows[r], b = row / p->n_q, i = row % p->n_q;
    int H = p->Hidx, D = p->d_idx, bad = 0;
    double* out = c->out + r * (int64_t)p->n_kv;
    double* qd = (double*)malloc(sizeof(double) * (size_t)H * D);
    double* wd = (double*)malloc(sizeof(double) * (size_t)H);
    double* kd = (double*)malloc(sizeof(double) * (size_t)D);
    for (int h = 0; h < H; ++h) {
        for (int d = 0; d < D; ++d)
            qd[h * D + d] = dec(&c->q, b * c->q.s0 + i * c->q.s1 + h * c->q.s2 + d, &bad);
        wd[h] = dec(&c->w, b * c->w.s0 + i * c->w.s1 + h, &bad);
    }
    for (int j = 0; j < p->n_kv; ++j) {
        if (!visible(p, b, i, j)) { out[j] = -INFINITY; continue; }
        for (int d = 0; d < D; ++d) kd[d] = dec(&c->k, b * c->k.s0 + (int64_t)j * c->k.s1 + d, &bad);
        double r_ = 0.0;
        for (int h = 0; h < H; ++h) {
            double z = 0.0;
            for (int d = 0; d < D; ++d) z += qd[h * D + d] * kd[d];
            double relu = z > 0.0 ? z : 0.0;
            r_ += wd[h] * relu;
        }
        out[j] = r_;
    }
    free(qd); free(wd); free(kd);
    if (bad) c->bad = 1;
}

/* scores[r, j] for the listed flat rows (b*n_q + i); -inf where not visible.
 * Returns 0, or -2 if a decoded input element is not finite. */
int or_scores(const or_problem* p, or_view q_idx, or_view k_idx, or_view w, int64_t nrows,
              const int32_t* rows, double* scores, int nthreads) {
    score_ctx c = {p, q_idx, k_idx, w, rows, scores, 0};
    pool_run(score_row, &c, nrows, nthreads);
    return c.bad ? -2 : 0;
}

/* --------------------------------------------------------------- select */

typedef struct { double s; int32_t pos, slot; } cand_t;

static int by_score_then_pos(const void* a_, const void* b_) {
    const cand_t *a = (const cand_t*)a_, *b = (const cand_t*)b_;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

static int by_pos(const void* a_, const void* b_) {
    const cand_t *a = (const cand_t*)a_, *b = (const cand_t*)b_;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

typedef struct {
    const or_problem* p;
    const double* scores;
    const int32_t* rows;
    int32_t* idx;
    double *sk, *skp1;
    int32_t* nsel;
} sel_ctx;

static void select_row(void* c_, int64_t r) {
    sel_ctx* c = (sel_ctx*)c_;
    const or_problem* p = c->p;
    int row = c->rows[r], b = row / p->n_q, i = row % p->n_q;
    const double* s = c->scores + r * (int64_t)p->n_kv;
    cand_t* v = (cand_t*)malloc(sizeof(cand_t) * (size_t)(p->n_kv > 0 ? p->n_kv : 1));
    int n = 0;
    for (int j = 0; j < p->n_kv; ++j)
        if (visible(p, b, i, j)) { v[n].s = s[j]; v[n].pos = pos_of(p, b, j); v[n].slot = j; ++n; }
    qsort(v, (size_t)n, sizeof(cand_t), by_score_then_pos);
    int m = n < p->k ? n : p->k;
    c->sk[r] = m > 0 ? v[m - 1].s : NAN;
    c->skp1[r] = m < n ? v[m].s : -INFINITY;
    c->nsel[r] = m;
    qsort(v, (size_t)m, sizeof(cand_t), by_pos);
    int32_t* o = c->idx + r * (int64_t)p->k;
    for (int t = 0; t < p->k; ++t) o[t] = t < m ? v[t].slot : -1;
    free(v);
}

/* Selection from given scores (one row of n_kv doubles per listed row).  idx gets the
 * selected slots in ascending position order, -1 padded; sk / skp1 get the k-th and
 * (k+1)-th largest visible scores (NaN / -inf when they do not exist). */
void or_select(const or_problem* p, const double* scores, int64_t nrows, const int32_t* rows,
               int32_t* idx, double* sk, double* skp1, int32_t* nsel, int nthreads) {
    sel_ctx c = {p, scores, rows, idx, sk, skp1, nsel};
    pool_run(select_row, &c, nrows, nthreads);
}

/* ------------------------------------------------------------ attention */

typedef struct {
    const or_problem* p;
    or_view Q, K, V;
    const int32_t* idx;
    int64_t idx_stride;
    const int32_t* rows;
    double *O, *lse;
    int bad;
} att_ctx;

static void attend_row(void* c_, int64_t r) {
    att_ctx* c = (att_ctx*)c_;
    const or_problem* p = c->p;
    int row = c->rows[r], b = row / p->n_q, i = row % p->n_q, bad = 0;
    int Dk = p->d_qk, Dv = p->d_v, group = p->Hq / p->Hkv;
    const int32_t* ix = c->idx + r * c->idx_stride;
    double* qd = (double*)malloc(sizeof(double) * (size_t)Dk);
    double* lg = (double*)malloc(sizeof(double) * (size_t)(p->k > 0 ? p->k : 1));
    int32_t* use = (int32_t*)malloc(sizeof(int32_t) * (size_t)(p->k > 0 ? p->k : 1));
    int n = 0;
    for (int t = 0; t < p->k; ++t) {
        int j = ix[t];
        if (j >= 0 && j < p->n_kv && visible(p, b, i, j)) use[n++] = j;
    }
    for (int hq = 0; hq < p->Hq; ++hq) {
        int hk = hq / group;
        double* O = c->O + (r * (int64_t)p->Hq + hq) * Dv;
        if (n == 0) {
            for (int d = 0; d < Dv; ++d) O[d] = 0.0;
            c->lse[r * (int64_t)p->Hq + hq] = -INFINITY;
            continue;
        }
        for (int d = 0; d < Dk; ++d) qd[d] = dec(&c->Q, b * c->Q.s0 + hq * c->Q.s1 + i * c->Q.s2 + d, &bad);
        double m = -INFINITY;
        for (int t = 0; t < n; ++t) {
            int64_t base = b * c->K.s0 + hk * c->K.s1 + (int64_t)use[t] * c->K.s2;
            double z = 0.0;
            for (int d = 0; d < Dk; ++d) z += qd[d] * dec(&c->K, base + d, &bad);
            lg[t] = p->scale * z;
            if (lg[t] > m) m = lg[t];
        }
        double Z = 0.0;
        for (int t = 0; t < n; ++t) Z += exp(lg[t] - m);
        for (int d = 0; d < Dv; ++d) O[d] = 0.0;
        for (int t = 0; t < n; ++t) {
            double pj = exp(lg[t] - m) / Z;
            int64_t base = b * c->V.s0 + hk * c->V.s1 + (int64_t)use[t] * c->V.s2;
            for (int d = 0; d < Dv; ++d) O[d] += pj * dec(&c->V, base + d, &bad);
        }
        c->lse[r * (int64_t)p->Hq + hq] = m + log(Z);
    }
    free(qd); free(lg); free(use);
    if (bad) c->bad = 1;
}

/* Softmax attention of the listed rows over the slots in idx (row r at idx + r*idx_stride,
 * p->k entries; -1, out-of-range and non-visible entries are skipped).
 * O: [nrows, Hq, d_v], lse: [nrows, Hq].  Returns -2 on a non-finite input. */
int or_attend(const or_problem* p, or_view Q, or_view K, or_view V, const int32_t* idx,
              int64_t idx_stride, int64_t nrows, const int32_t* rows, double* O, double* lse,
              int nthreads) {
    att_ctx c = {p, Q, K, V, idx, idx_stride, rows, O, lse, 0};
    pool_run(attend_row, &c, nrows, nthreads);
    return c.bad ? -2 : 0;
}

int or_version(void) { return 1; }
