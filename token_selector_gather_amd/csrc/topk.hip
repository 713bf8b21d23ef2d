// Per-row top-k selection.
//
// S(b,i) = the first min(k, L) visible positions in (score desc, position asc) order,
// written in ascending position; the remaining slots are -1 ("PaperTrace 2.2 ·
// Fine-grained indexing", §2.1: Select over the visible history, rows shorter than k
// return all their positions and mark the rest invalid; §3.1: lexicographic
// (score, index) order, NaN handled before the selection).
//
// One workgroup of 256 threads per row.  Scores map to order-preserving uint32 keys
// (sign-flip; -0 is folded onto +0).  A three-digit MSB radix select (11 + 11 + 10 bits,
// LDS histograms, one suffix scan per digit) finds the k-th largest key T and how many
// keys equal to T the set needs.  A final ordered pass then keeps every key > T and the
// first `need` keys == T in position order.  Each thread handles four consecutive
// positions per tile and a single packed block scan yields, for every position, both the
// number of greater keys and the number of equal keys before it, so the output is written
// in ascending position and exact ties go to the lower positions.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one uint32 per thread over the block; returns the prefix, sets total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wid] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        uint32_t t = wave_tot[w];
        if (w < wid) before += t;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

// Find the digit bin holding the `need`-th largest key among the histogram's entries.
// bins: NB counters.  Returns bin and number of entries in strictly higher bins.
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t need, uint32_t* wave_tot, int* out_bin,
                                         uint32_t* out_above) {
    constexpr int PER = NB / kThreads;  // bins per thread, highest bins to thread 0
    const int t = threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) local += hist[NB - 1 - (t * PER + e)];
    uint32_t total;
    uint32_t above = block_exclusive_scan(local, wave_tot, total);
    if (above < need && above + local >= need) {
        uint32_t run = above;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int bin = NB - 1 - (t * PER + e);
            const uint32_t c = hist[bin];
            if (run + c >= need) {
                *out_bin = bin;
                *out_above = run;
                break;
            }
            run += c;
        }
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kThreads) topk_rows(TopkArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wave_tot[kThreads / 64];
    __shared__ int s_bin;
    __shared__ uint32_t s_above;
    __shared__ int s_bad;

    const sa_problem& p = a.p;
    const int row = blockIdx.x;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const float* sc = a.scores + (int64_t)row * a.row_stride;
    int32_t* out = a.idx + (int64_t)row * K;
    float* vout = a.vals ? a.vals + (int64_t)row * K : nullptr;
    const int t = threadIdx.x;
    if (t == 0) {
        s_bad = 0;
        s_bin = 0;
        s_above = 0;
    }
    __syncthreads();

    if (L <= K) {
        int bad = 0;
        for (int j = t; j < K; j += kThreads) {
            float v = j < L ? sc[j] : -INFINITY;
            if (j < L && !isfinite(v)) bad = 1;
            out[j] = j < L ? j : -1;
            if (vout) vout[j] = v;
        }
        if (bad) s_bad = 1;
        __syncthreads();
        if (t == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
        return;
    }

    // ---- digit 1: bits 31..21
    for (int e = t; e < 2048; e += kThreads) hist[e] = 0;
    __syncthreads();
    int bad = 0;
    for (int j = t; j < L; j += kThreads) {
        float v = sc[j];
        if (!isfinite(v)) bad = 1;
        atomicAdd(&hist[order_key(v) >> 21], 1u);
    }
    if (bad) s_bad = 1;
    __syncthreads();
    find_bin<2048>(hist, (uint32_t)K, wave_tot, &s_bin, &s_above);
    const uint32_t d1 = (uint32_t)s_bin;
    uint32_t above = s_above;

    // ---- digit 2: bits 20..10 among keys with digit 1 == d1
    for (int e = t; e < 2048; e += kThreads) hist[e] = 0;
    __syncthreads();
    for (int j = t; j < L; j += kThreads) {
        uint32_t key = order_key(sc[j]);
        if ((key >> 21) == d1) atomicAdd(&hist[(key >> 10) & 2047u], 1u);
    }
    __syncthreads();
    find_bin<2048>(hist, (uint32_t)K - above, wave_tot, &s_bin, &s_above);
    const uint32_t d2 = (uint32_t)s_bin;
    above += s_above;

    // ---- digit 3: bits 9..0 among keys with digits 1,2 == d1,d2
    for (int e = t; e < 1024; e += kThreads) hist[e] = 0;
    __syncthreads();
    const uint32_t pre = (d1 << 11) | d2;
    for (int j = t; j < L; j += kThreads) {
        uint32_t key = order_key(sc[j]);
        if ((key >> 10) == pre) atomicAdd(&hist[key & 1023u], 1u);
    }
    __syncthreads();
    find_bin<1024>(hist, (uint32_t)K - above, wave_tot, &s_bin, &s_above);
    const uint32_t T = (pre << 10) | (uint32_t)s_bin;
    above += s_above;
    const uint32_t need_eq = (uint32_t)K - above;  // >= 1 keys equal to T to take

    // ---- ordered compaction
    uint32_t run_gt = 0, run_eq = 0;
    for (int base = 0; base < L; base += 4 * kThreads) {
        const int j0 = base + 4 * t;
        uint32_t keys[4];
        uint32_t c_gt = 0, c_eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + e;
            keys[e] = j < L ? order_key(sc[j]) : 0u;
            if (j < L) {
                c_gt += keys[e] > T;
                c_eq += keys[e] == T;
            }
        }
        uint32_t tot;
        const uint32_t pref = block_exclusive_scan(c_eq | (c_gt << 16), wave_tot, tot);
        uint32_t G = run_gt + (pref >> 16), E = run_eq + (pref & 0xffffu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + e;
            if (j >= L) break;
            const bool gt = keys[e] > T, eq = keys[e] == T;
            if (gt || (eq && E < need_eq)) {
                const uint32_t slot = G + (E < need_eq ? E : need_eq);
                if (slot < (uint32_t)K) {
                    out[slot] = j;
                    if (vout) vout[slot] = sc[j];
                }
            }
            G += gt;
            E += eq;
        }
        run_gt += tot >> 16;
        run_eq += tot & 0xffffu;
    }
    if (t == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
}

// ------------------------------------------------------------------ register path
// The same selection with NT threads and the row in registers: segments of VPT * NT
// positions, thread t holding positions c * 4NT + 4t .. 4t+3 of every chunk c of 4NT, all
// loaded with coalesced 16-byte loads.  A row of one segment is loaded once and every radix
// pass runs on registers; longer rows stream their segments through once per pass.  The
// ordered compaction walks the chunks in position order with one block scan each.

template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan_big(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wid] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        uint32_t t = wave_tot[w];
        if (w < wid) before += t;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

template <int NB, int NT>
__device__ __forceinline__ void find_bin_big(const uint32_t* hist, uint32_t need, uint32_t* wave_tot, int* out_bin,
                                             uint32_t* out_above) {
    constexpr int PER = NB / NT;  // bins per thread, highest bins to thread 0
    const int t = threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) local += hist[NB - 1 - (t * PER + e)];
    uint32_t total;
    const uint32_t above = block_exclusive_scan_big<NT>(local, wave_tot, total);
    if (above < need && above + local >= need) {
        uint32_t run = above;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int bin = NB - 1 - (t * PER + e);
            const uint32_t c = hist[bin];
            if (run + c >= need) {
                *out_bin = bin;
                *out_above = run;
                break;
            }
            run += c;
        }
    }
    __syncthreads();
}

// LDS histogram increment with lanes of the wave that share a bin combined first (scores
// of one row often crowd into a few bins of the leading digit, which would serialise plain
// atomics): up to four rounds pick the bin of the first remaining lane and add the
// population count of its matches; lanes still left then add individually.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    const int lane = threadIdx.x & 63;
    uint64_t rem = __ballot(active);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (rem == 0) break;
        const int leader = __ffsll((unsigned long long)rem) - 1;
        const uint32_t lb = __shfl(bin, leader);
        const uint64_t m = __ballot(active && bin == lb) & rem;
        if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(m));
        rem &= ~m;
    }
    if ((rem >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// keys of segment `seg` (positions >= L get key 0, below every real key); returns 1 on a
// non-finite visible score
template <int NCH, int NT>
__device__ __forceinline__ int load_segment(const float* sc, int L, int seg, bool vec_ok, uint32_t (&key)[NCH][4]) {
    int bad = 0;
    const int t = threadIdx.x;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j0 = (seg * NCH + c) * 4 * NT + 4 * t;
        float v[4];
        if (vec_ok && j0 + 3 < L) {
            const float4 f = *reinterpret_cast<const float4*>(sc + j0);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (j0 + e < L) ? sc[j0 + e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = j0 + e < L;
            if (in && !isfinite(v[e])) bad = 1;
            key[c][e] = in ? order_key(v[e]) : 0u;
        }
    }
    return bad;
}

template <int VPT, int NT>
__global__ void __launch_bounds__(NT) topk_rows_reg(TopkArgs a) {
    constexpr int NCH = VPT / 4;       // chunks of 4 * NT positions per segment
    constexpr int SEG = VPT * NT;    // positions per segment
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wave_tot[NT / 64];
    __shared__ int s_bin;
    __shared__ uint32_t s_above;
    __shared__ int s_bad;

    const sa_problem& p = a.p;
    const int row = blockIdx.x;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const float* sc = a.scores + (int64_t)row * a.row_stride;
    int32_t* out = a.idx + (int64_t)row * K;
    float* vout = a.vals ? a.vals + (int64_t)row * K : nullptr;
    const int t = threadIdx.x;
    if (t == 0) {
        s_bad = 0;
        s_bin = 0;
        s_above = 0;
    }
    __syncthreads();

    if (L <= K) {
        int bad = 0;
        for (int j = t; j < K; j += NT) {
            const float v = j < L ? sc[j] : -INFINITY;
            if (j < L && !isfinite(v)) bad = 1;
            out[j] = j < L ? j : -1;
            if (vout) vout[j] = v;
        }
        if (bad) s_bad = 1;
        __syncthreads();
        if (t == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
        return;
    }

    const bool vec_ok = ((a.row_stride & 3) == 0) && (((uintptr_t)a.scores & 15) == 0);
    const int nseg = (L + SEG - 1) / SEG;
    uint32_t key[NCH][4];
    if (nseg == 1 && load_segment<NCH, NT>(sc, L, 0, vec_ok, key)) s_bad = 1;

    // three MSB digits: 11, 11 and 10 bits; `above` counts keys in strictly higher bins
    uint32_t pre = 0, above = 0;
#pragma unroll 1
    for (int dgt = 0; dgt < 3; ++dgt) {
        const int shift = dgt == 0 ? 21 : (dgt == 1 ? 10 : 0);
        const uint32_t mask = dgt == 2 ? 1023u : 2047u;
        const int pshift = dgt == 0 ? 32 : shift + (dgt == 1 ? 11 : 10);
        for (int e = t; e < 2048; e += NT) hist[e] = 0;
        __syncthreads();
        for (int seg = 0; seg < nseg; ++seg) {
            if (nseg > 1 && load_segment<NCH, NT>(sc, L, seg, vec_ok, key) && dgt == 0) s_bad = 1;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kk = key[c][e];
                    const bool in = (seg * NCH + c) * 4 * NT + 4 * t + e < L;
                    const bool match = dgt == 0 ? true : ((uint32_t)((uint64_t)kk >> pshift) == pre);
                    hist_add(hist, (kk >> shift) & mask, in && match);
                }
        }
        __syncthreads();
        find_bin_big<2048, NT>(hist, (uint32_t)K - above, wave_tot, &s_bin, &s_above);
        // append this digit (11, 11 or 10 bits wide) to the prefix of the threshold key
        pre = dgt == 0 ? (uint32_t)s_bin : ((pre << (dgt == 1 ? 11 : 10)) | (uint32_t)s_bin);
        above += s_above;
    }
    const uint32_t T = pre;
    const uint32_t need_eq = (uint32_t)K - above;

    // ---- ordered compaction, segment by segment, chunk by chunk
    uint32_t run_gt = 0, run_eq = 0;
    for (int seg = 0; seg < nseg; ++seg) {
        if (nseg > 1) load_segment<NCH, NT>(sc, L, seg, vec_ok, key);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int cbase = (seg * NCH + c) * 4 * NT;
            if (cbase >= L) break;  // uniform
            const int j0 = cbase + 4 * t;
            uint32_t c_gt = 0, c_eq = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (j0 + e < L) {
                    c_gt += key[c][e] > T;
                    c_eq += key[c][e] == T;
                }
            }
            uint32_t tot;
            const uint32_t pref = block_exclusive_scan_big<NT>(c_eq | (c_gt << 16), wave_tot, tot);
            uint32_t G = run_gt + (pref >> 16), E = run_eq + (pref & 0xffffu);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + e;
                if (j >= L) break;
                const bool gt = key[c][e] > T, eq = key[c][e] == T;
                if (gt || (eq && E < need_eq)) {
                    const uint32_t slot = G + (E < need_eq ? E : need_eq);
                    if (slot < (uint32_t)K) {
                        out[slot] = j;
                        if (vout) vout[slot] = sc[j];
                    }
                }
                G += gt;
                E += eq;
            }
            run_gt += tot >> 16;
            run_eq += tot & 0xffffu;
        }
    }
    __syncthreads();
    if (t == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
    const long rows = (long)a.p.B * a.p.n_q;
    const int n = a.p.n_kv;
    const dim3 g((unsigned)rows);
    // short rows: 256 threads hold a whole row; long rows: 1024 threads, 32768-position segments
    if (n <= 1024) hipLaunchKernelGGL((topk_rows_reg<4, 256>), g, dim3(256), 0, s, a);
    else if (n <= 2048) hipLaunchKernelGGL((topk_rows_reg<8, 256>), g, dim3(256), 0, s, a);
    else if (n <= 4096) hipLaunchKernelGGL((topk_rows_reg<16, 256>), g, dim3(256), 0, s, a);
    else if (n <= 8192) hipLaunchKernelGGL((topk_rows_reg<32, 256>), g, dim3(256), 0, s, a);
    else if (n <= 16384) hipLaunchKernelGGL((topk_rows_reg<16, 1024>), g, dim3(1024), 0, s, a);
    else hipLaunchKernelGGL((topk_rows_reg<32, 1024>), g, dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
