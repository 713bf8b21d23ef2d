/*
 * Seeded synthetic input generator.
 *
 * This file produces the bytes that both the GPU library and the CPU oracle
 * consume: a counter-based random stream (splitmix64 finaliser over
 * (seed, tensor id, element index)), Box-Muller normals, uniforms, and the
 * storage encoders fp32 -> bf16 (round to nearest even) and
 * fp32 -> OCP FP8 e4m3fn (round to nearest even, saturating at +-448).
 *
 * It holds none of the method's arithmetic: no score, no selection, no
 * softmax.  Every element depends only on (seed, tensor id, flat index), so
 * any slice of any tensor can be regenerated independently and in parallel.
 *
 * Built with gcc as libsasynth.so; loaded through ctypes by sa_synth/__init__.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

enum { SYN_F32 = 0, SYN_BF16 = 1, SYN_E4M3 = 2, SYN_F64 = 3 };

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tid) {
    return mix64(seed * 0x9E3779B97F4A7C15ULL + tid * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL);
}

/* uniform double in [0,1) with 53 random bits */
static inline double u01(uint64_t key, uint64_t ctr) {
    uint64_t r = mix64(key + (ctr + 1) * 0x9E3779B97F4A7C15ULL);
    return (double)(r >> 11) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t e) {
    uint64_t p = e >> 1;
    double u1 = u01(key, 2 * p), u2 = u01(key, 2 * p + 1);
    double rad = sqrt(-2.0 * log(1.0 - u1));
    double th = 6.283185307179586476925 * u2;
    return (e & 1) ? rad * sin(th) : rad * cos(th);
}

static inline uint16_t enc_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0; /* NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* OCP e4m3fn: bias 7, no infinities, 0x7f/0xff are NaN, max finite 448. */
static inline uint8_t enc_e4m3(double v) {
    if (v != v) return 0x7f;
    uint8_t s = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return s | 0x7e;
    if (a < 0.015625) { /* below the smallest normal 2^-6: subnormal grid 2^-9 */
        double q = a * 512.0;
        double fl = floor(q), fr = q - fl;
        uint32_t m = (uint32_t)fl;
        if (fr > 0.5 || (fr == 0.5 && (m & 1))) m++;
        return s | (uint8_t)m; /* m==8 lands exactly on the first normal code */
    }
    int E;
    frexp(a, &E); /* a = f * 2^E, f in [0.5,1) -> unbiased exponent E-1 */
    int ue = E - 1;
    double step = ldexp(1.0, ue - 3);
    double q = a / step; /* in [8,16) */
    double fl = floor(q), fr = q - fl;
    uint32_t m = (uint32_t)fl;
    if (fr > 0.5 || (fr == 0.5 && (m & 1))) m++;
    if (m == 16) { m = 8; ue++; }
    uint32_t code = (uint32_t)((ue + 7) << 3) | (m - 8);
    if (code > 0x7e) code = 0x7e;
    return s | (uint8_t)code;
}

static void store(void* out, int dtype, int64_t i, double v) {
    switch (dtype) {
    case SYN_F32: ((float*)out)[i] = (float)v; break;
    case SYN_BF16: ((uint16_t*)out)[i] = enc_bf16((float)v); break;
    case SYN_E4M3: ((uint8_t*)out)[i] = enc_e4m3((double)(float)v); break;
    default: ((double*)out)[i] = v; break;
    }
}

typedef struct {
    int kind; /* 0 normal, 1 uniform, 2 encode */
    uint64_t key;
    int64_t off, lo_i, hi_i;
    double a, b;
    int dtype;
    void* out;
    const double* in;
} job_t;

static void* run_job(void* arg) {
    job_t* j = (job_t*)arg;
    for (int64_t i = j->lo_i; i < j->hi_i; ++i) {
        double v;
        if (j->kind == 0) v = j->a * normal_at(j->key, (uint64_t)(j->off + i)) + j->b;
        else if (j->kind == 1) v = j->a + (j->b - j->a) * u01(j->key, (uint64_t)(j->off + i));
        else v = j->in[i];
        store(j->out, j->dtype, i, v);
    }
    return 0;
}

static void run_parallel(job_t proto, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n < 65536) nthreads = 1;
    pthread_t th[64];
    job_t jobs[64];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].lo_i = t * chunk;
        jobs[t].hi_i = (t + 1) * chunk < n ? (t + 1) * chunk : n;
        if (jobs[t].lo_i >= jobs[t].hi_i) break;
        if (nthreads == 1) { run_job(&jobs[t]); started = 0; break; }
        pthread_create(&th[t], 0, run_job, &jobs[t]);
        started = t + 1;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], 0);
}

/* out[i] = scale * N(0,1)[off+i] + shift, encoded as dtype. */
void syn_normal(uint64_t seed, uint64_t tid, int64_t off, int64_t n, double scale, double shift,
                int dtype, void* out, int nthreads) {
    job_t p = {0};
    p.kind = 0; p.key = stream_key(seed, tid); p.off = off; p.a = scale; p.b = shift;
    p.dtype = dtype; p.out = out;
    run_parallel(p, n, nthreads);
}

/* out[i] = lo + (hi-lo) * U[0,1)[off+i], encoded as dtype. */
void syn_uniform(uint64_t seed, uint64_t tid, int64_t off, int64_t n, double lo, double hi,
                 int dtype, void* out, int nthreads) {
    job_t p = {0};
    p.kind = 1; p.key = stream_key(seed, tid); p.off = off; p.a = lo; p.b = hi;
    p.dtype = dtype; p.out = out;
    run_parallel(p, n, nthreads);
}

/* Encode n doubles into dtype storage. */
void syn_encode(const double* in, int64_t n, int dtype, void* out, int nthreads) {
    job_t p = {0};
    p.kind = 2; p.in = in; p.dtype = dtype; p.out = out;
    run_parallel(p, n, nthreads);
}

int syn_version(void) { return 1; }
