// Per-row top-k selection.
//
// S(b,i) = the first min(k, L) visible positions in (score desc, position asc) order,
// written in ascending position; the remaining slots are -1 ("PaperTrace 2.2 ·
// Fine-grained indexing", §2.1: Select over the visible history, rows shorter than k
// return all their positions and mark the rest invalid; §3.1: lexicographic
// (score, index) order, NaN handled before the selection).
//
// Three layouts: one workgroup per row with the row in registers (up to 8192 positions:
// 256 threads; 8193 to 32768: 1024 threads, first digit relative to the row's own key range
// and the threshold bin resolved from an LDS list), and several workgroups per row for a few
// long rows (decode batches).  The description below is the register path.
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

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
    const int row = a.row0 + (int)blockIdx.x;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const float* sc = a.scores + (int64_t)(row - a.row0) * a.row_stride;
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
                    if (in && match) atomicAdd(&hist[(kk >> shift) & mask], 1u);
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

// ---------------------------------------------------------------- long-row path
// Rows of 8193 to 32768 positions, one workgroup of NT threads per row, the row in registers
// (thread t holds positions 4 NT c + 4t .. 4t + 3 of every chunk c).  The first digit is taken
// relative to the row's own key range: bin = (key - kmin) >> s with s chosen so that
// (kmax - kmin) >> s < 2048, which spreads concentrated scores over the histogram.  The keys
// of the threshold bin are then gathered into LDS and the remaining s bits are resolved there
// (at most two more 11-bit digits); a bin too large for the list is resolved over the
// registers instead.  The ordered write uses per-(chunk, wave) counts, one scan over them and
// ballots inside each wave, so a chunk costs no block-wide scan.
template <int NT, int NCH>
__global__ void __launch_bounds__(NT) topk_rows_long(TopkArgs a) {
    constexpr int NW = NT / 64, CAP = 4096;
    static_assert(NCH * NW <= 128, "the (chunk, wave) scan takes two entries per lane");
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t cand[CAP];
    __shared__ uint32_t wave_tot[NW];
    __shared__ uint32_t cnt[NCH * NW][2];  // per (chunk, wave): keys > T, keys == T; then exclusive prefixes
    __shared__ uint32_t s_min[NW], s_max[NW];
    __shared__ int s_bin;
    __shared__ uint32_t s_above, s_ncand;
    __shared__ int s_bad;

    const sa_problem& p = a.p;
    const int row = a.row0 + (int)blockIdx.x;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const float* sc = a.scores + (int64_t)(row - a.row0) * a.row_stride;
    int32_t* out = a.idx + (int64_t)row * K;
    float* vout = a.vals ? a.vals + (int64_t)row * K : nullptr;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    if (t == 0) {
        s_bad = 0;
        s_bin = 0;
        s_above = 0;
        s_ncand = 0;
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

    // keys (0 past L, below every real key: a visible key is never 0, the bit pattern that
    // would map to 0 is a NaN, which is reported) and the row's key range
    const bool vec_ok = ((a.row_stride & 3) == 0) && (((uintptr_t)a.scores & 15) == 0);
    const int nch = min(NCH, (L + 4 * NT - 1) / (4 * NT));  // chunks holding visible positions
    uint32_t key[NCH][4];
    int bad = 0;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j0 = c * 4 * NT + 4 * t;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (c < nch) {
            if (vec_ok && j0 + 3 < L) {
                const float4 f = *reinterpret_cast<const float4*>(sc + j0);
                v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (j0 + e < L) ? sc[j0 + e] : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = j0 + e < L;
            if (in && !isfinite(v[e])) bad = 1;
            key[c][e] = in ? order_key(v[e]) : 0u;
            kmin = min(kmin, key[c][e] != 0u ? key[c][e] : 0xffffffffu);
            kmax = max(kmax, key[c][e]);
        }
    }
    if (bad) s_bad = 1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if (lane == 0) {
        s_min[wv] = kmin;
        s_max[wv] = kmax;
    }
    for (int e = t; e < 2048; e += NT) hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kmin = min(kmin, s_min[w]);
        kmax = max(kmax, s_max[w]);
    }
    const uint32_t range = kmax - kmin;
    const int sh = range == 0 ? 0 : max(0, 32 - __clz((int)range) - 11);  // (key - kmin) >> sh < 2048

    // first digit
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c >= nch) break;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (key[c][e] != 0u) atomicAdd(&hist[(key[c][e] - kmin) >> sh], 1u);
    }
    __syncthreads();
    find_bin_big<2048, NT>(hist, (uint32_t)K, wave_tot, &s_bin, &s_above);
    const uint32_t B = (uint32_t)s_bin;
    uint32_t above = s_above;
    const uint32_t nB = hist[B];
    uint32_t tu = B << sh;  // threshold relative to kmin, refined below
    if (sh > 0) {
        // gather the keys of bin B (relative to kmin) when they fit the list
        const bool listed = nB <= (uint32_t)CAP;
        if (listed) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (c >= nch) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t u = key[c][e] - kmin;
                    const bool hit = key[c][e] != 0u && (u >> sh) == B;
                    const uint64_t m = __ballot(hit);
                    if (m == 0) continue;
                    uint32_t base = 0;
                    if (lane == 0) base = atomicAdd(&s_ncand, (uint32_t)__popcll(m));
                    base = __shfl(base, 0);
                    if (hit) cand[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = u;
                }
            }
        }
        // A short list (the usual case: tens of keys) is ranked by one wave: candidate c is the
        // threshold when fewer than `need` candidates exceed it and at least `need` are >= it.
        // Longer lists and unlisted bins take at most two more digits over the low sh bits.
        int done = 0;  // low bits still open: sh - done
        if (listed && nB <= 64u) {
            __syncthreads();  // list complete
            if (wv == 0) {
                const uint32_t need = (uint32_t)K - above;
                const uint32_t c = lane < (int)nB ? cand[lane] : 0u;
                uint32_t g = 0, q = 0;
                for (uint32_t j = 0; j < nB; ++j) {
                    const uint32_t cj = cand[j];
                    g += cj > c;
                    q += cj == c;
                }
                const bool hit = lane < (int)nB && g < need && need <= g + q;
                const uint64_t m = __ballot(hit);
                const int src = __builtin_ctzll(m);  // a threshold always exists; equal values agree
                const uint32_t cu = __shfl(c, src), gu = __shfl(g, src);
                if (lane == 0) {
                    s_bin = (int)cu;
                    s_above = gu;
                }
            }
            __syncthreads();
            tu = (uint32_t)s_bin;  // the full key relative to kmin
            above += s_above;
            done = sh;
        }
        while (done < sh) {
            const int wdt = min(11, sh - done);
            const int dsh = sh - done - wdt;
            const uint32_t pmask_shift = (uint32_t)(sh - done);  // bits above the digit already fixed
            const uint32_t prefix = tu >> pmask_shift;
            __syncthreads();  // list complete / previous histogram read
            for (int e = t; e < 2048; e += NT) hist[e] = 0;
            __syncthreads();
            if (listed) {
                for (uint32_t q = t; q < nB; q += NT) {
                    const uint32_t u = cand[q];
                    if ((u >> pmask_shift) == prefix) atomicAdd(&hist[(u >> dsh) & ((1u << wdt) - 1u)], 1u);
                }
            } else {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    if (c >= nch) break;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t u = key[c][e] - kmin;
                        if (key[c][e] != 0u && (u >> pmask_shift) == prefix)
                            atomicAdd(&hist[(u >> dsh) & ((1u << wdt) - 1u)], 1u);
                    }
                }
            }
            __syncthreads();
            if (t == 0) s_bin = 0, s_above = 0;
            __syncthreads();
            find_bin_big<2048, NT>(hist, (uint32_t)K - above, wave_tot, &s_bin, &s_above);
            tu |= (uint32_t)s_bin << dsh;
            above += s_above;
            done += wdt;
        }
    }
    const uint32_t T = kmin + tu;
    const uint32_t need_eq = (uint32_t)K - above;

    // ordered write: counts per (chunk, wave), one exclusive scan in (chunk, wave) order, then
    // ballot prefixes inside each wave
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        uint32_t g = 0, q = 0;
        if (c < nch) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // T is a visible key, so neither test holds for a position past L (key 0)
                g += (uint32_t)__popcll(__ballot(key[c][e] > T));
                q += (uint32_t)__popcll(__ballot(key[c][e] == T));
            }
        }
        if (lane == 0) {
            cnt[c * NW + wv][0] = g;
            cnt[c * NW + wv][1] = q;
        }
    }
    __syncthreads();
    if (wv == 0) {
        // NCH * NW <= 128 entries, two per lane
        uint32_t g0 = 0, q0 = 0, g1 = 0, q1 = 0;
        const int e0 = 2 * lane, e1 = 2 * lane + 1;
        if (e0 < NCH * NW) { g0 = cnt[e0][0]; q0 = cnt[e0][1]; }
        if (e1 < NCH * NW) { g1 = cnt[e1][0]; q1 = cnt[e1][1]; }
        uint32_t gs = g0 + g1, qs = q0 + q1;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t gy = __shfl_up(gs, o), qy = __shfl_up(qs, o);
            if (lane >= o) { gs += gy; qs += qy; }
        }
        const uint32_t gb = gs - g0 - g1, qb = qs - q0 - q1;  // exclusive
        if (e0 < NCH * NW) { cnt[e0][0] = gb; cnt[e0][1] = qb; }
        if (e1 < NCH * NW) { cnt[e1][0] = gb + g0; cnt[e1][1] = qb + q0; }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c >= nch) break;
        const int j0 = c * 4 * NT + 4 * t;
        uint32_t G = cnt[c * NW + wv][0], E = cnt[c * NW + wv][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            G += (uint32_t)__popcll(__ballot(key[c][e] > T) & below);
            E += (uint32_t)__popcll(__ballot(key[c][e] == T) & below);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool gt = key[c][e] > T, eq = key[c][e] == T;
            if (gt || (eq && E < need_eq)) {
                const uint32_t slot = G + (E < need_eq ? E : need_eq);
                if (slot < (uint32_t)K) {
                    out[slot] = j0 + e;
                    if (vout) vout[slot] = sc[j0 + e];
                }
            }
            G += gt;
            E += eq;
        }
    }
    __syncthreads();
    if (t == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
}

// -------------------------------------------------------------------- sliced path
// Few long rows (decode batches): each row is cut into slices of 4096 positions with one
// 256-thread workgroup per slice, so 8 or 64 rows still occupy the whole GPU.  The radix
// select above runs as a short chain of kernels with per-row digit histograms in the
// workspace, accumulated atomically by the row's workgroups; each kernel re-derives the
// threshold prefix from the finished histograms of the earlier digits.  The last two
// kernels count keys > T and == T per slice (the count kernel also writes the rows with
// L <= k) and compact in position order, each slice starting after the counts of the row's
// earlier slices.  Inside a selection the index scan adds the first digit while it writes the
// scores (digit0_done: the histograms are cleared before the scan, and the first histogram
// kernel is skipped).
constexpr int kSlice = 4096, kSliceT = 256;

struct SlicedWs {
    uint32_t* hist;    // [rows][3][2048]
    uint32_t* counts;  // [rows][S][2]  (greater, equal)
    uint32_t* state;   // [rows][4]     (T, need_eq)
    int S;
};

__device__ __forceinline__ void load_slice16(const float* sc, int L, int j0, bool vec_ok, uint32_t (&key)[4][4],
                                             int& bad) {
    const int t = threadIdx.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = j0 + c * 4 * kSliceT + 4 * t;
        float v[4];
        if (vec_ok && j + 3 < L) {
            const float4 f = *reinterpret_cast<const float4*>(sc + j);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (j + e < L) ? sc[j + e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = j + e < L;
            if (in && !isfinite(v[e])) bad = 1;
            key[c][e] = in ? order_key(v[e]) : 0u;
        }
    }
}

// prefix of the threshold after `ndig` digits and the count of keys above it
__device__ __forceinline__ void sliced_prefix(const uint32_t* ghist, int ndig, uint32_t K, uint32_t* lh,
                                              uint32_t* wave_tot, int* s_bin, uint32_t* s_above, uint32_t& pre,
                                              uint32_t& above) {
    pre = 0;
    above = 0;
    for (int dgt = 0; dgt < ndig; ++dgt) {
        for (int e = threadIdx.x; e < 2048; e += kSliceT) lh[e] = ghist[dgt * 2048 + e];
        __syncthreads();
        find_bin_big<2048, kSliceT>(lh, K - above, wave_tot, s_bin, s_above);
        pre = dgt == 0 ? (uint32_t)*s_bin : ((pre << (dgt == 1 ? 11 : 10)) | (uint32_t)*s_bin);
        above += *s_above;
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256) topk_sl_zero(SlicedWs w, long words) {
    for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < words; e += (long)gridDim.x * 256) w.hist[e] = 0;
}

template <int DIGIT>
__global__ void __launch_bounds__(kSliceT) topk_sl_hist(TopkArgs a, SlicedWs w) {
    __shared__ uint32_t lh[2048];
    __shared__ uint32_t wave_tot[kSliceT / 64];
    __shared__ int s_bin;
    __shared__ uint32_t s_above;
    __shared__ int s_bad;
    const sa_problem& p = a.p;
    const int row = blockIdx.x / w.S, slice = blockIdx.x % w.S;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const int j0 = slice * kSlice;
    const float* sc = a.scores + (int64_t)row * a.row_stride;
    if (threadIdx.x == 0) { s_bad = 0; s_bin = 0; s_above = 0; }
    __syncthreads();
    if (L <= K || j0 >= L) return;  // (short rows are written by topk_sl_count)
    uint32_t* gh = w.hist + (int64_t)row * 3 * 2048;
    uint32_t pre, above;
    sliced_prefix(gh, DIGIT, (uint32_t)K, lh, wave_tot, &s_bin, &s_above, pre, above);
    for (int e = threadIdx.x; e < 2048; e += kSliceT) lh[e] = 0;
    __syncthreads();
    uint32_t key[4][4];
    int bad = 0;
    const bool vec_ok = ((a.row_stride & 3) == 0) && (((uintptr_t)a.scores & 15) == 0);
    load_slice16(sc, L, j0, vec_ok, key, bad);
    const int shift = DIGIT == 0 ? 21 : (DIGIT == 1 ? 10 : 0);
    const uint32_t mask = DIGIT == 2 ? 1023u : 2047u;
    const int pshift = DIGIT == 1 ? 21 : 10;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = j0 + c * 4 * kSliceT + 4 * threadIdx.x + e < L;
            const bool match = DIGIT == 0 ? true : ((key[c][e] >> pshift) == pre);
            if (in && match) atomicAdd(&lh[(key[c][e] >> shift) & mask], 1u);
        }
    if (DIGIT == 0 && bad) s_bad = 1;
    __syncthreads();
    for (int e = threadIdx.x; e < 2048; e += kSliceT)
        if (lh[e]) atomicAdd(&gh[DIGIT * 2048 + e], lh[e]);
    if (DIGIT == 0 && threadIdx.x == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
}

// per-slice counts of keys greater than / equal to the threshold T
__global__ void __launch_bounds__(kSliceT) topk_sl_count(TopkArgs a, SlicedWs w) {
    __shared__ uint32_t lh[2048];
    __shared__ uint32_t wave_tot[kSliceT / 64];
    __shared__ int s_bin;
    __shared__ uint32_t s_above;
    const sa_problem& p = a.p;
    const int row = blockIdx.x / w.S, slice = blockIdx.x % w.S;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const int j0 = slice * kSlice;
    if (L <= K) {  // short row: all visible positions, then -1
        __shared__ int s_bad;
        const float* sc = a.scores + (int64_t)row * a.row_stride;
        int32_t* out = a.idx + (int64_t)row * K;
        float* vout = a.vals ? a.vals + (int64_t)row * K : nullptr;
        if (threadIdx.x == 0) s_bad = 0;
        __syncthreads();
        int bad = 0;
        for (int j = j0 + threadIdx.x; j < min(K, j0 + kSlice) || (slice == w.S - 1 && j < K); j += kSliceT) {
            const float v = j < L ? sc[j] : -INFINITY;
            if (j < L && !isfinite(v)) bad = 1;
            out[j] = j < L ? j : -1;
            if (vout) vout[j] = v;
        }
        if (bad) s_bad = 1;
        __syncthreads();
        if (threadIdx.x == 0 && s_bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
        return;
    }
    if (threadIdx.x == 0) { s_bin = 0; s_above = 0; }
    __syncthreads();
    uint32_t* gh = w.hist + (int64_t)row * 3 * 2048;
    uint32_t T, above;
    sliced_prefix(gh, 3, (uint32_t)K, lh, wave_tot, &s_bin, &s_above, T, above);
    if (slice == 0 && threadIdx.x == 0) {
        w.state[row * 4 + 0] = T;
        w.state[row * 4 + 1] = (uint32_t)K - above;
    }
    uint32_t gt = 0, eq = 0;
    if (j0 < L) {
        uint32_t key[4][4];
        int bad = 0;
        const bool vec_ok = ((a.row_stride & 3) == 0) && (((uintptr_t)a.scores & 15) == 0);
        load_slice16(a.scores + (int64_t)row * a.row_stride, L, j0, vec_ok, key, bad);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j0 + c * 4 * kSliceT + 4 * threadIdx.x + e < L) {
                    gt += key[c][e] > T;
                    eq += key[c][e] == T;
                }
    }
    uint32_t tot;
    block_exclusive_scan_big<kSliceT>(eq | (gt << 16), wave_tot, tot);
    if (threadIdx.x == 0) {
        w.counts[((int64_t)row * w.S + slice) * 2 + 0] = tot >> 16;
        w.counts[((int64_t)row * w.S + slice) * 2 + 1] = tot & 0xffffu;
    }
}

// ordered compaction: slice s writes after the greater/equal counts of slices < s
__global__ void __launch_bounds__(kSliceT) topk_sl_compact(TopkArgs a, SlicedWs w) {
    __shared__ uint32_t wave_tot[kSliceT / 64];
    __shared__ uint32_t s_g0, s_e0;
    const sa_problem& p = a.p;
    const int row = blockIdx.x / w.S, slice = blockIdx.x % w.S;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int K = p.k;
    const int j0 = slice * kSlice;
    if (L <= K || j0 >= L) return;
    const uint32_t T = w.state[row * 4 + 0], need_eq = w.state[row * 4 + 1];
    if (threadIdx.x < 64) {
        uint32_t g = 0, e = 0;
        for (int s2 = threadIdx.x; s2 < slice; s2 += 64) {
            g += w.counts[((int64_t)row * w.S + s2) * 2 + 0];
            e += w.counts[((int64_t)row * w.S + s2) * 2 + 1];
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            g += __shfl_xor(g, o);
            e += __shfl_xor(e, o);
        }
        if (threadIdx.x == 0) { s_g0 = g; s_e0 = e; }
    }
    __syncthreads();
    const float* sc = a.scores + (int64_t)row * a.row_stride;
    int32_t* out = a.idx + (int64_t)row * K;
    float* vout = a.vals ? a.vals + (int64_t)row * K : nullptr;
    uint32_t key[4][4];
    int bad = 0;
    const bool vec_ok = ((a.row_stride & 3) == 0) && (((uintptr_t)a.scores & 15) == 0);
    load_slice16(sc, L, j0, vec_ok, key, bad);
    uint32_t run_gt = s_g0, run_eq = s_e0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int jc = j0 + c * 4 * kSliceT + 4 * threadIdx.x;
        uint32_t c_gt = 0, c_eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (jc + e < L) {
                c_gt += key[c][e] > T;
                c_eq += key[c][e] == T;
            }
        uint32_t tot;
        const uint32_t pref = block_exclusive_scan_big<kSliceT>(c_eq | (c_gt << 16), wave_tot, tot);
        uint32_t G = run_gt + (pref >> 16), E = run_eq + (pref & 0xffffu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = jc + e;
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

}  // namespace

bool topk_sliced(const sa_problem& p) { return (long)p.B * p.n_q <= 512 && p.n_kv > 8192; }

uint32_t* topk_sliced_hist(const TopkArgs& a) { return static_cast<uint32_t*>(a.scratch); }

hipError_t topk_sliced_clear(const TopkArgs& a, hipStream_t s) {
    if (!topk_sliced(a.p) || a.nrows > 0) return hipErrorInvalidValue;
    const long rows = (long)a.p.B * a.p.n_q, words = rows * 3 * 2048;
    SlicedWs w;
    w.hist = topk_sliced_hist(a);
    hipLaunchKernelGGL(topk_sl_zero, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, s, w, words);
    return hipGetLastError();
}

size_t topk_ws_bytes(const sa_problem& p) {
    if (!topk_sliced(p)) return 0;
    const long rows = (long)p.B * p.n_q;
    const long S = (p.n_kv + kSlice - 1) / kSlice;
    return (size_t)rows * (3 * 2048 + 2 * S + 4) * sizeof(uint32_t);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
    const long rows = a.nrows > 0 ? a.nrows : (long)a.p.B * a.p.n_q;
    const int n = a.p.n_kv;
    const dim3 g((unsigned)rows);
    if (topk_sliced(a.p)) {
        if (a.nrows > 0) return hipErrorInvalidValue;  // the sliced path takes whole problems
        SlicedWs w;
        w.S = (n + kSlice - 1) / kSlice;
        w.hist = static_cast<uint32_t*>(a.scratch);
        w.counts = w.hist + rows * 3 * 2048;
        w.state = w.counts + rows * 2 * w.S;
        const long words = rows * 3 * 2048;
        const dim3 gs((unsigned)(rows * w.S));
        if (!a.digit0_done) {  // (otherwise cleared and filled with the first digit already)
            hipLaunchKernelGGL(topk_sl_zero, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                               dim3(256), 0, s, w, words);
            hipLaunchKernelGGL(topk_sl_hist<0>, gs, dim3(kSliceT), 0, s, a, w);
        }
        hipLaunchKernelGGL(topk_sl_hist<1>, gs, dim3(kSliceT), 0, s, a, w);
        hipLaunchKernelGGL(topk_sl_hist<2>, gs, dim3(kSliceT), 0, s, a, w);
        hipLaunchKernelGGL(topk_sl_count, gs, dim3(kSliceT), 0, s, a, w);
        hipLaunchKernelGGL(topk_sl_compact, gs, dim3(kSliceT), 0, s, a, w);
        return hipGetLastError();
    }
    // short rows: 256 threads hold a whole row; long rows: 1024 threads, 32768-position segments
    if (n <= 1024) hipLaunchKernelGGL((topk_rows_reg<4, 256>), g, dim3(256), 0, s, a);
    else if (n <= 2048) hipLaunchKernelGGL((topk_rows_reg<8, 256>), g, dim3(256), 0, s, a);
    else if (n <= 4096) hipLaunchKernelGGL((topk_rows_reg<16, 256>), g, dim3(256), 0, s, a);
    else if (n <= 8192) hipLaunchKernelGGL((topk_rows_reg<32, 256>), g, dim3(256), 0, s, a);
    else if (n <= 16384) hipLaunchKernelGGL((topk_rows_long<1024, 4>), g, dim3(1024), 0, s, a);
    else if (n <= 32768) hipLaunchKernelGGL((topk_rows_long<1024, 8>), g, dim3(1024), 0, s, a);
    else hipLaunchKernelGGL((topk_rows_reg<32, 1024>), g, dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
