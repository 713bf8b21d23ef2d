/*
 * Host-code sanitizer driver (test infrastructure): builds a small seeded workload with the
 * input generator (sa_synth/synth.c) and runs the oracle's score, select and attend on it
 * with several threads, so that a build with -fsanitize=address,undefined checks both
 * host libraries for out-of-bounds accesses, leaks and undefined behaviour.  Prints a
 * checksum; exits non-zero on a failed call.
 *
 * The structs below mirror oracle.c's or_problem / or_view (the oracle's ABI).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int32_t B, n_q, n_kv, Hq, Hkv, d_qk, d_v, Hidx, d_idx, k, causal;
    double scale;
    const int32_t* kv_len;
    const int32_t* q_pos0;
    const int32_t* pos_of_slot;
} or_problem;

typedef struct {
    const void* data;
    int32_t dtype;
    int64_t s0, s1, s2;
} or_view;

int or_scores(const or_problem* p, or_view q_idx, or_view k_idx, or_view w, int64_t nrows, const int32_t* rows,
              double* scores, int nthreads);
void or_select(const or_problem* p, const double* scores, int64_t nrows, const int32_t* rows, int32_t* idx,
               double* sk, double* skp1, int32_t* nsel, int nthreads);
int or_attend(const or_problem* p, or_view Q, or_view K, or_view V, const int32_t* idx, int64_t idx_stride,
              int64_t nrows, const int32_t* rows, double* O, double* lse, int nthreads);
void syn_normal(uint64_t seed, uint64_t tid, int64_t off, int64_t n, double scale, double shift, int dtype, void* out,
                int nthreads);
void syn_uniform(uint64_t seed, uint64_t tid, int64_t off, int64_t n, double lo, double hi, int dtype, void* out,
                 int nthreads);

enum { F32 = 0, BF16 = 1, E4M3 = 2 };

static int run(int causal, int nthreads) {
    const int B = 2, nq = 40, nkv = 48, Hq = 4, Hkv = 2, dqk = 16, dv = 16, Hidx = 4, didx = 8, k = 6;
    int32_t kv_len[2] = {48, 29}, q_pos0[2] = {8, 0};
    or_problem p = {B, nq, nkv, Hq, Hkv, dqk, dv, Hidx, didx, k, causal, 0.25, kv_len, q_pos0, NULL};
    const int64_t nQ = (int64_t)B * Hq * nq * dqk, nK = (int64_t)B * Hkv * nkv * dqk, nV = (int64_t)B * Hkv * nkv * dv;
    const int64_t nqi = (int64_t)B * nq * Hidx * didx, nki = (int64_t)B * nkv * didx, nw = (int64_t)B * nq * Hidx;
    uint16_t* Q = malloc(sizeof(uint16_t) * nQ);
    uint16_t* K = malloc(sizeof(uint16_t) * nK);
    uint16_t* V = malloc(sizeof(uint16_t) * nV);
    uint16_t* qi = malloc(sizeof(uint16_t) * nqi);
    uint8_t* ki = malloc(nki);
    float* w = malloc(sizeof(float) * nw);
    syn_normal(7, 1, 0, nQ, 1.0, 0.0, BF16, Q, nthreads);
    syn_normal(7, 2, 0, nK, 1.0, 0.0, BF16, K, nthreads);
    syn_normal(7, 3, 0, nV, 1.0, 0.0, BF16, V, nthreads);
    syn_normal(7, 4, 0, nqi, 1.0, 0.0, BF16, qi, nthreads);
    syn_normal(7, 5, 0, nki, 1.0, 0.0, E4M3, ki, nthreads);
    syn_uniform(7, 6, 0, nw, -1.0, 1.0, F32, w, nthreads);

    const int64_t R = (int64_t)B * nq;
    int32_t* rows = malloc(sizeof(int32_t) * R);
    for (int64_t r = 0; r < R; ++r) rows[r] = (int32_t)r;
    double* sc = malloc(sizeof(double) * R * nkv);
    int32_t* idx = malloc(sizeof(int32_t) * R * k);
    double* sk = malloc(sizeof(double) * R);
    double* skp1 = malloc(sizeof(double) * R);
    int32_t* nsel = malloc(sizeof(int32_t) * R);
    double* O = malloc(sizeof(double) * R * Hq * dv);
    double* lse = malloc(sizeof(double) * R * Hq);
    or_view vq = {qi, BF16, (int64_t)nq * Hidx * didx, (int64_t)Hidx * didx, didx};
    or_view vk = {ki, E4M3, (int64_t)nkv * didx, didx, 0};
    or_view vw = {w, F32, (int64_t)nq * Hidx, Hidx, 0};
    or_view VQ = {Q, BF16, (int64_t)Hq * nq * dqk, (int64_t)nq * dqk, dqk};
    or_view VK = {K, BF16, (int64_t)Hkv * nkv * dqk, (int64_t)nkv * dqk, dqk};
    or_view VV = {V, BF16, (int64_t)Hkv * nkv * dv, (int64_t)nkv * dv, dv};
    int rc = or_scores(&p, vq, vk, vw, R, rows, sc, nthreads);
    if (rc == 0) or_select(&p, sc, R, rows, idx, sk, skp1, nsel, nthreads);
    if (rc == 0) rc = or_attend(&p, VQ, VK, VV, idx, k, R, rows, O, lse, nthreads);
    double sum = 0.0;
    for (int64_t e = 0; e < R * Hq * dv; ++e) sum += O[e];
    for (int64_t e = 0; e < R * k; ++e) sum += idx[e];
    printf("causal %d threads %d rc %d checksum %.12g\n", causal, nthreads, rc, sum);
    free(Q); free(K); free(V); free(qi); free(ki); free(w); free(rows); free(sc); free(idx); free(sk);
    free(skp1); free(nsel); free(O); free(lse);
    return rc;
}

int main(void) {
    int rc = 0;
    rc |= run(1, 1);
    rc |= run(1, 3);
    rc |= run(0, 2);
    return rc != 0;
}
