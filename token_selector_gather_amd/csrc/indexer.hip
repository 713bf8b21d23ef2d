// Indexer score kernels.
//
// r[b,i,j] = sum_h w[b,i,h] * ReLU(<q_idx[b,i,h,:], k_idx[b,j,:]>)  for visible j
// ("PaperTrace 2.2 · Fine-grained indexing", §1.1 and §3.2: per-query index heads, one
// index key per token shared by all heads, query-dependent head weights).
//
// Matrix-core paths (bf16 index queries; bf16 or OCP-e4m3 index keys).  The contraction
// is a GEMM with M = (query, index head) rows, N = history positions, K = d_idx, on
// v_mfma_f32_16x16x32_bf16; e4m3 keys widen to bf16 exactly in hardware
// (v_cvt_scalef32_pk_bf16_fp8, scale 1).  The epilogue applies ReLU and the head weights to
// the fp32 accumulators and sums the heads inside the accumulator layout (in-lane, then
// lane swaps between rows), in the same order for every position j: byte-identical keys
// get bit-identical scores.  Three layouts:
//  * indexer_pf: many query rows (prefill); a workgroup walks the causal history of a block
//    of rows once, keys widened to bf16 once per LDS chunk;
//  * indexer_dec: few query rows (decode); the waves split the keys of one row;
//  * indexer_mfma3: the remaining shapes (4 or 8 index heads, moderate row counts).
// indexer_valu covers f32 inputs and other widths.
//
// Non-finite index inputs must reach the selection's finiteness check instead of being
// clipped to zero by the ReLU: the VALU path uses (z > 0 ? z : 0*z); the matrix-core paths
// use a one-instruction integer-max ReLU and either add z * 0 to each score, check the
// inputs in a pre-pass (fused call), or mark rows and keys with non-finite inputs apart.
#include <algorithm>

#include "gfx950_mem.h"
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float relu_keep_nonfinite(float z) { return z > 0.f ? z : 0.f * z; }
// ReLU in one integer max: negative floats are negative int32 patterns (-0 included),
// non-negative floats keep their pattern.  Exact for finite values; +inf and positive NaN
// pass, -inf and negative NaN give 0.  A kernel that may see non-finite dot products either
// adds z * 0 (0, or NaN for a non-finite z) to the score, or its launcher marks the rows and
// keys with non-finite inputs separately (indexer_pf without the pre-pass).
__device__ __forceinline__ float relu_finite(float z) { return __int_as_float(max(__float_as_int(z), 0)); }
__device__ __forceinline__ bool bf16x2_nonfinite(uint32_t w) {
    return ((w & 0x7f80u) == 0x7f80u) || ((w & 0x7f800000u) == 0x7f800000u);
}
__device__ __forceinline__ bool e4m3x4_nan(uint32_t w) {
    const uint32_t t = w & 0x7f7f7f7fu;            // a byte is 0x7f exactly when adding 1
    return ((t + 0x01010101u) & 0x80808080u) != 0;  // carries into its top bit
}

// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] by lane swaps between rows (no LDS round trip)
__device__ __forceinline__ float xsum16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float xsum32(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ float load_elem(const void* base, int dtype, int64_t e) {
    if (dtype == SA_F32) return static_cast<const float*>(base)[e];
    if (dtype == SA_BF16) {
        uint32_t u = (uint32_t) static_cast<const uint16_t*>(base)[e] << 16;
        return __uint_as_float(u);
    }
    uint32_t c = static_cast<const uint8_t*>(base)[e];
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
    return v[0];
}

// ---------------------------------------------------------------- plain VALU path
// One block = one query row x 256 positions.  The query's index vectors and weights are
// widened to fp32 in LDS; every thread scores one position.
__global__ void __launch_bounds__(256) indexer_valu(IndexerArgs a) {
    extern __shared__ float smem[];
    const sa_problem& p = a.p;
    const int row = a.row0 + (int)blockIdx.x;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int j = blockIdx.y * 256 + threadIdx.x;
    float* out = a.scores + (int64_t)(row - a.row0) * a.row_stride;
    if ((int)(blockIdx.y * 256) >= L) {
        if (a.fill_invisible && j < p.n_kv) out[j] = -INFINITY;
        return;
    }
    const int H = p.Hidx, D = p.d_idx;
    float* qs = smem;
    float* ws = smem + H * D;
    for (int t = threadIdx.x; t < H * D; t += 256) {
        int h = t / D, d = t % D;
        qs[t] = load_elem(a.q.data, a.q.dtype, b * a.q.s0 + i * a.q.s1 + h * a.q.s2 + d);
    }
    for (int t = threadIdx.x; t < H; t += 256) ws[t] = static_cast<const float*>(a.w.data)[b * a.w.s0 + i * a.w.s1 + t];
    __syncthreads();
    if (j >= p.n_kv) return;
    if (j >= L) {
        if (a.fill_invisible) out[j] = -INFINITY;
        return;
    }
    const int64_t kb = b * a.k.s0 + (int64_t)j * a.k.s1;
    float r = 0.f;
    for (int h = 0; h < H; ++h) {
        float z = 0.f;
        for (int d = 0; d < D; ++d) z = fmaf(qs[h * D + d], load_elem(a.k.data, a.k.dtype, kb + d), z);
        r = fmaf(ws[h], relu_keep_nonfinite(z), r);
    }
    out[j] = r;
}

// ------------------------------------------------------------- matrix-core path
constexpr int kChunk = 256;  // positions per wave
constexpr int kMT = 4;       // 16-row M-tiles per wave (64 rows)



// ------------------------------------------------------------------ indexer_dec
// Few query rows (decode): a workgroup takes one query row and a range of at most 2048 keys;
// each wave holds all H index heads of that row (H / 16 M-tiles) and walks its own 16-key
// tiles of the range (tile u of wave w covers keys 16 (w + 4 u)), so every key is widened
// once and no wave waits for another.  Tiles reach a ring of NB slots in the wave's own LDS
// region through buffer loads that write LDS directly (NB - 1 tiles in flight per wave, no
// staging registers, ordered by the wave's own vmcnt waits); scores collect in LDS and are
// stored once per workgroup.  The contraction index is relabelled so that lane group g owns
// d in [g D/4, (g+1) D/4): each lane's share of a key row is one contiguous piece (the Q
// fragments use the same relabelling).
template <int KSTEPS, bool KE4M3, int H, bool FAST_RELU>
__global__ void __launch_bounds__(256, 4) indexer_dec(IndexerArgs a, int n_rng, int rng_len) {
    static_assert(H >= 16 && H <= 64, "whole 16-row M-tiles of one query");
    constexpr int MT = H / 16;
    constexpr int RB = 32 * KSTEPS * (KE4M3 ? 1 : 2);  // bytes per key row
    constexpr int KB = RB / 4;                         // bytes of a key row per lane group
    constexpr int NV = KB / 16;                        // 16-byte pieces per lane per tile
    constexpr int CPR = RB / 16;                       // 16-byte chunks per key row
    constexpr int TB = 16 * RB;                        // bytes per 16-key tile
    constexpr int NI = TB / 1024;                      // LDS-direct loads per tile
    constexpr int RPI = 1024 / RB;                     // key rows per load
    constexpr int NB = 8192 / TB < 4 ? 4 : 8192 / TB;  // ring slots per wave (8 KB for 2 KB tiles)
    static_assert(NI >= 1 && NI * 1024 == TB && NI * (NB - 1) < 64, "tile and ring sizes");
    constexpr int MAXR = 2048;                         // keys per workgroup range
    __shared__ __attribute__((aligned(16))) uint8_t ring[4 * NB * TB];
    __shared__ float s_sc[MAXR];

    const sa_problem& p = a.p;
    const int lane = threadIdx.x & 63, l15 = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long wg = blockIdx.x;
    const int rng = (int)(wg % n_rng);
    const long row = wg / n_rng;  // b * n_q + i
    const int b = (int)(row / p.n_q), i = (int)(row % p.n_q);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const int L = visible_len(R, b, i);
    const int j_begin = rng * rng_len, j_end = min(j_begin + rng_len, p.n_kv);
    const int j_comp = min(j_end, L);  // keys worth computing: [j_begin, j_comp)
    const int ntl = j_comp > j_begin ? (j_comp - j_begin + 15) / 16 : 0;  // tiles of the range
    const int nmine = ntl > wv ? (ntl - wv + 3) / 4 : 0;                  // tiles of this wave
    // within a key row, chunk c sits in slot c ^ cswz(r): conflict-free 16-row fragment reads
    auto cswz = [](int r) { return (r / (16 / CPR < 1 ? 1 : 16 / CPR)) & (CPR - 1); };

    if (nmine > 0) {
        // A fragments: row 16 m + lane%16 = head, k-step s holds d = g D/4 + 8 s + 0..7
        bf16x8 av[MT][KSTEPS];
        float wvv[MT][4];
        const uint16_t* qp = static_cast<const uint16_t*>(a.q.data) + b * a.q.s0 + (int64_t)i * a.q.s1;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                av[m][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + (16 * m + l15) * a.q.s2 + 8 * KSTEPS * g + 8 * s));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wvv[m][e] = static_cast<const float*>(a.w.data)[b * a.w.s0 + (int64_t)i * a.w.s1 + 16 * m + 4 * g + e];
        }
        wait_vmcnt<0>();  // the tile loop's waits count tile loads only
        const uint32_t kstride = (uint32_t)(a.k.s1 * (KE4M3 ? 1 : 2));
        const v4i krs = buffer_rsrc(static_cast<const uint8_t*>(a.k.data) + b * a.k.s0 * (KE4M3 ? 1 : 2), (uint32_t)j_comp * kstride);
        const uint32_t ring_w = lds_addr(ring) + (uint32_t)(wv * NB * TB);
        // this lane's row and chunk in load ii of a tile
        int lrow[NI];
        uint32_t loff[NI];
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
            lrow[ii] = ii * RPI + lane / CPR;
            loff[ii] = (uint32_t)lrow[ii] * kstride + 16u * (uint32_t)((lane % CPR) ^ cswz(lrow[ii]));
        }
        auto issue = [&](int u) {
            const int j0 = j_begin + 16 * (wv + 4 * u);
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) {
                const bool ok = u < nmine && j0 + lrow[ii] < j_comp;
                lds_dma16(krs, ring_w + (uint32_t)((u % NB) * TB + 1024 * ii), ok ? (uint32_t)j0 * kstride + loff[ii] : 0x80000000u, 0u);
            }
        };
#pragma unroll
        for (int u = 0; u < NB - 1; ++u) issue(u);
        const uint8_t* rbase = ring + wv * NB * TB + l15 * RB;
        for (int u = 0; u < nmine; ++u) {
            issue(u + NB - 1);       // into the slot of tile u - 1, whose reads fed the MFMAs already
            wait_vmcnt<NI * (NB - 1)>();  // tile u has landed
            const uint8_t* tr = rbase + (u % NB) * TB;
            uint4 rr[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) rr[v] = *reinterpret_cast<const uint4*>(tr + 16 * ((NV * g + v) ^ cswz(l15)));
            bf16x8 bv[KSTEPS];
            if constexpr (KE4M3) {
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    const uint4 w4 = rr[s / 2];
                    const uint32_t lo = (s & 1) ? w4.z : w4.x, hi = (s & 1) ? w4.w : w4.y;
                    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
                    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
                    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
                    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
                    bv[s] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                }
            } else {
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) bv[s] = __builtin_bit_cast(bf16x8, rr[s]);
            }
            f32x4 acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][s], bv[s], acc[m], 0, 0, 0);
            // four partial sums; z * 0 keeps every non-finite dot product visible in the score
            float t[4] = {0.f, 0.f, 0.f, 0.f}, chk = 0.f;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t[e] = fmaf(wvv[m][e], relu_finite(acc[m][e]), t[e]);
                    if (!FAST_RELU) chk = fmaf(acc[m][e], 0.f, chk);
                }
            const float tt = (t[0] + t[1]) + (t[2] + t[3]);
            const float v = xsum32(xsum16(FAST_RELU ? tt : tt + chk));
            if (lane < 16) s_sc[16 * (wv + 4 * u) + l15] = v;
        }
        wait_vmcnt<0>();
    }
    __syncthreads();
    // store the range: computed keys that are visible, -inf for the rest when asked to
    float* srow = a.scores + row * a.row_stride;
    for (int j = j_begin + (int)threadIdx.x; j < j_end; j += 256) {
        const bool vis = j < L;
        if (vis) srow[j] = s_sc[j - j_begin];
        else if (a.fill_invisible) srow[j] = -INFINITY;
    }
    if (a.hist0 != nullptr && j_comp > j_begin) {  // (uniform)
        // the first radix digit (top 11 bits of the order-preserving key, -0 folded onto +0) of
        // this range's visible scores, into the row's histogram of the sliced top-k
        uint32_t* lh = reinterpret_cast<uint32_t*>(ring);  // (the tile ring is free now)
        for (int e = threadIdx.x; e < 2048; e += 256) lh[e] = 0u;
        __syncthreads();
        int bad = 0;
        for (int j = j_begin + (int)threadIdx.x; j < j_comp; j += 256) {
            const float v = s_sc[j - j_begin];
            uint32_t u = __float_as_uint(v);
            if ((u & 0x7fffffffu) == 0) u = 0;
            const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
            bad |= !isfinite(v);
            atomicAdd(&lh[key >> 21], 1u);
        }
        __syncthreads();
        uint32_t* gh = a.hist0 + row * (int64_t)(3 * 2048);
        for (int e = threadIdx.x; e < 2048; e += 256)
            if (lh[e]) atomicAdd(&gh[e], lh[e]);
        if (__ballot(bad) != 0 && lane == 0 && a.status) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
    }
}

// ------------------------------------------------------------ streaming selection
// The fused score + select of the many-row layout keeps, per query row, a list of candidate
// (key, position) pairs in the workgroup's own slice of the workspace instead of the row's
// scores ("PaperTrace 2.2 · Fine-grained indexing", §2.1: score the history slice by slice,
// keep local candidates and merge down to k; the result is the global top-k).  Keys are the
// order-preserving uint32 images of the fp32 scores (-0 folded onto +0).  A score enters the
// list only if its key is above the row's threshold tau, and the list stays in position
// order (ballot ranks inside a tile, tiles in order).
//
// tau stays below the k-th largest key seen so far, so every key that can still be in the
// row's top k is in the list (a key at or below tau has k larger keys before it).  It is
// raised from a histogram of the list's keys kept in LDS: after the first chunk the row's
// scores fix the bins (uniform in score, see below; bin 0 below the first boundary, the last
// bin open above), every append adds its score, and tau becomes the key of the lower
// boundary of the bin that holds the k-th largest listed key, minus one.  When the list could overflow at
// the next chunk, the keys at or below tau are dropped (one ordered pass; the bins below
// tau's bin empty exactly).  If that frees too little (keys far outside the bins), the list
// is cut to its exact top k and the bins are rebuilt around the cut.  At the end the exact
// k-th key comes from the histogram and digits of its bin, and one ordered pass writes the
// selection.  Passes over a list issue their loads in batches, so a pass costs a few
// memory round trips.

__device__ __forceinline__ uint32_t sel_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// The smallest score whose key is above tau (key > tau <=> score >= sel_floor(tau), NaN
// aside), so the hot loop compares floats and computes keys only for appended scores.
__device__ __forceinline__ float sel_floor(uint32_t tau) {
    if (tau == 0u) return -INFINITY;  // nothing is cut yet
    const uint32_t k = tau + 1u;
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// threadIdx.x through an opaque move: values derived from it are recomputed where they are
// used instead of being hoisted out of the persistent loop and kept live across the MFMA loop
__device__ __forceinline__ int opaque_tid() {
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
    return t;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Cross-lane steps on DPP (no LDS round trip): row shifts with zero fill, row broadcasts,
// quad / half-row / row mirrors.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, true);
}
// wave-wide exclusive prefix sum and total: inclusive scans inside each 16-lane row by
// shifts of 1, 2, 4 and 8, then row 0's total into rows 1 and 3 and rows 0-1's into 2 and 3
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t x, int lane, uint32_t& total) {
    (void)lane;
    uint32_t incl = x;
    incl += dpp_u32<0x111>(incl);       // row_shr:1
    incl += dpp_u32<0x112>(incl);       // row_shr:2
    incl += dpp_u32<0x114>(incl);       // row_shr:4
    incl += dpp_u32<0x118>(incl);       // row_shr:8
    incl += dpp_u32<0x142, 0xa>(incl);  // row_bcast:15
    incl += dpp_u32<0x143, 0xc>(incl);  // row_bcast:31
    total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    return incl - x;
}
// wave-uniform minimum / maximum: inside each row by mirrors, then the four rows' lanes
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));
    const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Bins of a row's histogram, uniform in score: with a power-of-two width W = 2^e and an
// integer origin j0, bin 0 holds the scores below j0 W, bin b in [1, NB - 1) the scores in
// [(j0 + b - 1) W, (j0 + b) W), bin NB - 1 everything above.  Bins uniform in the score keep
// their resolution where a row's scores change sign (bins uniform in the key would spend
// themselves on the tiny magnitudes around zero).  Exactness: every boundary (j0 + b - 1) W
// is a float (|j0| + NB < 2^24 and e in [-126, 103]), and floor(v / W) is exact (v 2^-e is
// exact when |v| >= W, and |v| < W is decided by a comparison), so a key lies in a bin >= b
// exactly when it is at least the key of that bin's lower boundary.  The row's bin state
// is (W as float bits, j0).
__device__ __forceinline__ float sel_val(uint32_t key) {  // inverse of sel_key (+0 for a folded -0)
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}
__device__ __forceinline__ float sel_ffloor(float v, uint32_t wbits) {  // floor(v / W)
    const float W = __uint_as_float(wbits);
    const float Wi = __uint_as_float((254u - (wbits >> 23)) << 23);  // 2^-e
    return fabsf(v) < W ? (v < 0.f ? -1.f : 0.f) : floorf(v * Wi);
}
template <int NB>
__device__ __forceinline__ int sel_bin(float v, uint32_t wbits, int j0) {
    const float x = sel_ffloor(v, wbits) - (float)j0 + 1.f;
    return (int)fminf(fmaxf(x, 0.f), (float)(NB - 1));
}
__device__ __forceinline__ uint32_t bin_lowest(int b, uint32_t wbits, int j0) {  // b >= 1: key of the lower boundary
    return sel_key((float)(j0 + b - 1) * __uint_as_float(wbits));
}
// bins for keys spanning [lo, hi]: the span takes at most NB / 2 bins (the rest is room
// above), the width is at least 2^-22 of the larger magnitude (|j0| < 2^23)
template <int NB>
__device__ __forceinline__ void sel_bins(uint32_t lo, uint32_t hi, uint32_t& wbits, int& j0) {
    const float vlo = sel_val(lo), vhi = sel_val(hi);
    const float span = (vhi - vlo) * (1.f / (float)(NB / 2 - 1));
    const int ex_span = span > 0.f ? (int)((__float_as_uint(fminf(span, 3.0e38f)) >> 23) & 0xff) - 127 + 1 : -126;
    const float mag = fminf(fmaxf(fabsf(vlo), fabsf(vhi)), 3.0e38f);
    const int ex_mag = (int)((__float_as_uint(mag) >> 23) & 0xff) - 127 - 22;
    const int e = min(max(max(ex_span, ex_mag), -126), 103);
    wbits = (uint32_t)(e + 127) << 23;
    const float f = fminf(fmaxf(sel_ffloor(vlo, wbits), -8388608.f), 8388608.f);
    j0 = (int)f;
}

// In an NB-bin histogram (bins ascending in key), the bin holding the need-th largest
// counted key and the number of keys in higher bins (need <= total).  Lane l reads bins
// NB - 1 - 4 l down to NB - 4 - 4 l.
template <int NB>
__device__ __forceinline__ void sel_find_bin(const uint32_t* h, uint32_t need, int lane, int& bin, uint32_t& above) {
    static_assert(NB % 4 == 0 && NB <= 256, "four bins per lane");
    uint4 c = make_uint4(0u, 0u, 0u, 0u);
    if (4 * lane < NB) c = *reinterpret_cast<const uint4*>(h + NB - 4 - 4 * lane);
    const uint32_t cnt[4] = {c.w, c.z, c.y, c.x};  // bins NB - 1 - 4 lane - e, e = 0 .. 3
    const uint32_t local = c.x + c.y + c.z + c.w;
    uint32_t total;
    const uint32_t excl = wave_excl_scan(local, lane, total);
    int bl = 0;
    uint32_t ab = 0, run = excl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (bl == 0 && run + cnt[e] >= need) {
            bl = NB - 4 * lane - e;  // bin + 1
            ab = run;
        }
        run += cnt[e];
    }
    const uint64_t m = __ballot(excl < need && excl + local >= need);
    const int src = m ? __builtin_ctzll(m) : 0;
    bin = max(__builtin_amdgcn_readlane(bl, src) - 1, 0);
    above = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
}

// The same search for four rows at once, one per 16-lane group (h: the group's histogram):
// lane l of a group reads bins NB - 1 - BPL l down to NB - BPL (l + 1), the group scans
// inside its DPP row, and every lane of the group gets the bin (0 when need exceeds the
// total).
template <int NB>
__device__ __forceinline__ int sel_find_bin_rows(const uint32_t* h, uint32_t need, int l15) {
    constexpr int BPL = (NB + 15) / 16;
    uint32_t cnt[BPL], local = 0;
#pragma unroll
    for (int e = 0; e < BPL; ++e) {
        const int b = NB - 1 - BPL * l15 - e;
        cnt[e] = b >= 0 ? h[b] : 0u;
        local += cnt[e];
    }
    uint32_t incl = local;
    incl += dpp_u32<0x111>(incl);  // row_shr:1
    incl += dpp_u32<0x112>(incl);  // row_shr:2
    incl += dpp_u32<0x114>(incl);  // row_shr:4
    incl += dpp_u32<0x118>(incl);  // row_shr:8
    uint32_t run = incl - local;
    uint32_t bl = 0;  // bin + 1 on the lane where the count crosses need
#pragma unroll
    for (int e = 0; e < BPL; ++e) {
        if (bl == 0 && run < need && run + cnt[e] >= need) bl = (uint32_t)(NB - BPL * l15 - e);
        run += cnt[e];
    }
    // maximum over the row: quad swaps, half-row mirror, row mirror
    bl = max(bl, (uint32_t)__builtin_amdgcn_update_dpp((int)bl, (int)bl, 0xB1, 0xf, 0xf, false));
    bl = max(bl, (uint32_t)__builtin_amdgcn_update_dpp((int)bl, (int)bl, 0x4E, 0xf, 0xf, false));
    bl = max(bl, (uint32_t)__builtin_amdgcn_update_dpp((int)bl, (int)bl, 0x141, 0xf, 0xf, false));
    bl = max(bl, (uint32_t)__builtin_amdgcn_update_dpp((int)bl, (int)bl, 0x140, 0xf, 0xf, false));
    return bl > 0 ? (int)bl - 1 : 0;
}

// Scratch of one wave for exact thresholds: a 256-bin digit histogram and a short list.
struct SelScratch {
    uint32_t hist[256];
    uint32_t list[64];
};

constexpr int kSelU = 8;  // 16-byte loads per lane in flight in a pass over a list

// A batch of up to kSelU x 256 keys from entry e0 (lane: 4 consecutive keys per load).
__device__ __forceinline__ void sel_load(const uint32_t* keys, int n, int e0, int lane, uint4 (&v)[kSelU]) {
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
        const int e = e0 + 256 * u + 4 * lane;
        if (e + 3 < n) {
            v[u] = *reinterpret_cast<const uint4*>(keys + e);
        } else {
            v[u].x = e < n ? keys[e] : 0u;
            v[u].y = e + 1 < n ? keys[e + 1] : 0u;
            v[u].z = e + 2 < n ? keys[e + 2] : 0u;
            v[u].w = e + 3 < n ? keys[e + 3] : 0u;
        }
    }
}

// Exact threshold of the top `need` keys among the keys of [lo, top] (nB of them, all in
// [lo, lo + 2^bits)), refining the digit below `bits` (a 256-bin histogram per step, or the
// short list once the open bin holds at most 64 keys).  tu: relative prefix so far.
// Returns T and the number of keys equal to T that the selection keeps.
__device__ __forceinline__ void sel_refine(const uint32_t* keys, int n, uint32_t lo, uint32_t top, int bits, uint32_t tu,
                                           uint32_t nB, uint32_t need, SelScratch* sc, int lane, uint32_t& T,
                                           uint32_t& need_eq) {
    while (bits > 0) {
        if (nB <= 64u) {
            // the open bin's keys to a list, ranked by one lane each
            const uint32_t pref = (uint32_t)((uint64_t)tu >> bits);
            uint32_t cntl = 0;
            for (int e0 = 0; e0 < n; e0 += 256 * kSelU) {
                uint4 v[kSelU];
                sel_load(keys, n, e0, lane, v);
#pragma unroll
                for (int u = 0; u < kSelU; ++u) {
                    const int e = e0 + 256 * u + 4 * lane;
                    const uint32_t k4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    bool hit[4];
                    uint32_t c = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hit[i] = e + i < n && k4[i] >= lo && k4[i] <= top && (uint32_t)((uint64_t)(k4[i] - lo) >> bits) == pref;
                        c += hit[i];
                    }
                    uint32_t tot;
                    uint32_t at = cntl + wave_excl_scan(c, lane, tot);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (hit[i]) sc->list[at++] = k4[i] - lo;
                    cntl += tot;
                }
            }
            wait_lgkmcnt0();
            const uint32_t c = lane < (int)nB ? sc->list[lane] : 0u;
            uint32_t gt = 0, eq = 0;
            for (uint32_t t = 0; t < nB; ++t) {
                const uint32_t ct = sc->list[t];
                gt += ct > c;
                eq += ct == c;
            }
            const uint64_t m = __ballot(lane < (int)nB && gt < need && need <= gt + eq);
            const int src = m ? __builtin_ctzll(m) : 0;
            tu = (uint32_t)__builtin_amdgcn_readlane((int)c, src);
            need -= (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
            bits = 0;
            break;
        }
        const int d = bits < 8 ? bits : 8;
        bits -= d;
        const uint32_t pref = (uint32_t)((uint64_t)tu >> (bits + d)), dmask = (1u << d) - 1u;
        *reinterpret_cast<uint4*>(sc->hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        for (int e0 = 0; e0 < n; e0 += 256 * kSelU) {
            uint4 v[kSelU];
            sel_load(keys, n, e0, lane, v);
#pragma unroll
            for (int u = 0; u < kSelU; ++u) {
                const int e = e0 + 256 * u + 4 * lane;
                const uint32_t k4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t r = k4[i] - lo;
                    if (e + i < n && k4[i] >= lo && k4[i] <= top && (uint32_t)((uint64_t)r >> (bits + d)) == pref)
                        atomicAdd(&sc->hist[(r >> bits) & dmask], 1u);
                }
            }
        }
        wait_lgkmcnt0();
        int bin;
        uint32_t above;
        sel_find_bin<256>(sc->hist, need, lane, bin, above);
        nB = sc->hist[bin];
        tu |= (uint32_t)bin << bits;
        need -= above;
    }
    T = lo + tu;
    need_eq = need;
}

// Exact threshold of the top K of n keys (K < n) with no other information: the key range
// (a pass), then the refinement over the whole range.  Also returns the largest key.
__device__ __forceinline__ void sel_threshold(const uint32_t* keys, int n, uint32_t K, SelScratch* sc, int lane,
                                              uint32_t& T, uint32_t& need_eq, uint32_t& hi) {
    uint32_t lo = 0xffffffffu;
    hi = 0u;
    for (int e0 = 0; e0 < n; e0 += 256 * kSelU) {
        uint4 v[kSelU];
        sel_load(keys, n, e0, lane, v);
#pragma unroll
        for (int u = 0; u < kSelU; ++u) {
            const int e = e0 + 256 * u + 4 * lane;
            const uint32_t k4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < n) {
                    lo = min(lo, k4[i]);
                    hi = max(hi, k4[i]);
                }
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    const uint32_t range = hi - lo;
    const int bits = range == 0 ? 0 : 32 - __clz((int)range);  // every key has (key - lo) >> bits == 0
    sel_refine(keys, n, lo, hi, bits, 0u, (uint32_t)n, K, sc, lane, T, need_eq);
}

// Ordered compaction of a list: keeps the entries with key > T and the first need_eq
// entries with key == T (T = 0xffffffff with need_eq = 0 is never used: keys > T do not
// exist), writing them to (okeys, opos) -- which may be the source arrays -- or only the
// positions when okeys is null.  Returns the number kept.
__device__ __forceinline__ uint32_t sel_compact(uint32_t* keys, int32_t* pos, int n, uint32_t T, uint32_t need_eq,
                                                uint32_t* okeys, int32_t* opos, int lane) {
    constexpr int U = kSelU / 2;
    uint32_t run_gt = 0, run_eq = 0;
    for (int e0 = 0; e0 < n; e0 += 256 * U) {
        uint4 kv[U], pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + 256 * u + 4 * lane;
            if (e + 3 < n) {
                kv[u] = *reinterpret_cast<const uint4*>(keys + e);
                pv[u] = *reinterpret_cast<const uint4*>(pos + e);
            } else {
                kv[u].x = e < n ? keys[e] : 0u;
                kv[u].y = e + 1 < n ? keys[e + 1] : 0u;
                kv[u].z = e + 2 < n ? keys[e + 2] : 0u;
                kv[u].w = e + 3 < n ? keys[e + 3] : 0u;
                pv[u].x = e < n ? pos[e] : 0;
                pv[u].y = e + 1 < n ? pos[e + 1] : 0;
                pv[u].z = e + 2 < n ? pos[e + 2] : 0;
                pv[u].w = e + 3 < n ? pos[e + 3] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + 256 * u + 4 * lane;
            const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
            const int32_t p4[4] = {(int32_t)pv[u].x, (int32_t)pv[u].y, (int32_t)pv[u].z, (int32_t)pv[u].w};
            uint32_t cg = 0, ce = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cg += e + i < n && k4[i] > T;
                ce += e + i < n && k4[i] == T;
            }
            uint32_t tot;
            const uint32_t ex = wave_excl_scan(cg | (ce << 16), lane, tot);
            uint32_t G = run_gt + (ex & 0xffffu), E = run_eq + (ex >> 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool gt = e + i < n && k4[i] > T, eq = e + i < n && k4[i] == T;
                if (gt || (eq && E < need_eq)) {
                    const uint32_t slot = G + (E < need_eq ? E : need_eq);
                    if (okeys) okeys[slot] = k4[i];
                    opos[slot] = p4[i];
                }
                G += gt;
                E += eq;
            }
            run_gt += tot & 0xffffu;
            run_eq += tot >> 16;
        }
    }
    return run_gt + (run_eq < need_eq ? run_eq : need_eq);
}

// ------------------------------------------------------------------ indexer_pf

// Prefill layout for many query rows: a workgroup takes QB = 4 * 128 / H consecutive query
// rows of one batch and walks their causal history once, in chunks of 128 keys that are
// widened to bf16 once per chunk while being written to LDS (double buffered).  Wave w
// keeps the A fragments of its 128 (query, head) rows (eight 16-row M-tiles) in registers,
// so each 16-key B fragment read from LDS feeds 8 x KSTEPS MFMAs, and the ReLU /
// head-weighting / head-sum arithmetic is about 2.5 VALU instructions per MFMA.
// SEL: the fused score + select.  The grid is persistent (at most kSelSlots workgroups,
// each with its own candidate lists); workgroup w takes the blocks of rows w, 2G - 1 - w,
// 2G + w, ... of the list ordered by history length (G = grid size), which evens out the
// causal triangle.  Scores are not stored: each lane group appends its query's scores
// above the row threshold to the row's candidate list and histogram (see the streaming
// selection above); at chunk boundaries each wave raises its rows' thresholds and drops
// dead entries when a list is nearly full, and at the end it writes the selection.  The
// non-finite check of the index inputs is done on the way (query fragments, weights, and
// each key chunk as it is widened) and reported in the status word.
template <int KSTEPS, bool KE4M3, int H, bool SEL>
__global__ void __launch_bounds__(256, 2) indexer_pf(IndexerArgs a, int n_qb, SelectArgs sel) {
    static_assert(H >= 16 && H <= 64, "one query per 16-row M-tile");
    constexpr int D = 32 * KSTEPS;
    constexpr int QW = 128 / H;              // queries per wave
    constexpr int QB = 4 * QW;               // queries per workgroup
    constexpr int MT = 8;                    // 16-row M-tiles per wave
    constexpr int TPQ = H / 16;              // M-tiles per query
    constexpr int CK = 128;                  // keys per chunk
    constexpr int KP = 2 * D + 16;           // LDS pitch of one widened key row (bytes)
    constexpr int RB = D * (KE4M3 ? 1 : 2);  // bytes per key row in memory
    constexpr int PPR = RB / 16;             // 16-byte pieces per key row
    constexpr int PPT = CK * PPR / 256;      // pieces per thread per chunk
    constexpr int NZ = QW > 4 ? 2 : 1;       // queries per lane group
    static_assert(PPT >= 1 && PPT * 256 == CK * PPR, "chunk pieces must split evenly over the threads");
    // SEL: per-row key histograms in the LDS left for two workgroups per CU
    constexpr int NBR0 = ((81920 - 2 * CK * KP - 64 - 4 * (int)sizeof(SelScratch)) / QB - 8) / 4;
    constexpr int NBR = NBR0 >= 256 ? 256 : (NBR0 / 16) * 16;
    static_assert(!SEL || NBR >= 32, "row histograms");
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][CK * KP];
    __shared__ int s_L[QB];
    __shared__ __attribute__((aligned(16))) SelScratch s_sel[SEL ? 4 : 1];
    __shared__ __attribute__((aligned(16))) uint32_t s_rh[SEL ? QB : 1][SEL ? NBR : 4];  // row histograms
    __shared__ uint32_t s_rp[SEL ? QB : 1][2];                                         // bins: base, shift

    const sa_problem& p = a.p;
    const int lane = threadIdx.x & 63, l15 = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long n_items = (long)p.B * n_qb;
    const int K = p.k;
    bool bad_input = false;  // SEL: a non-finite index input this thread saw

    for (long rnd = 0;; ++rnd) {
    long wg;
    int b, qb;
    if constexpr (SEL) {
        const long base = rnd * (long)gridDim.x;
        if (base >= n_items) break;
        wg = base + ((rnd & 1) ? (long)gridDim.x - 1 - (long)blockIdx.x : (long)blockIdx.x);
        if (wg >= n_items) continue;
        // batches interleaved so that the list runs from the longest histories down
        const long r = wg / p.B;
        b = (int)(wg % p.B);
        qb = p.causal ? n_qb - 1 - (int)r : (int)r;
        __syncthreads();  // the previous block's readers of s_L are done
    } else {
        if (rnd > 0) break;
        wg = blockIdx.x;
        qb = p.causal ? n_qb - 1 - (int)(wg % n_qb) : (int)(wg % n_qb);  // longest histories first
        b = (int)(wg / n_qb);
    }
    const int i0 = qb * QB;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    if (threadIdx.x < QB) s_L[threadIdx.x] = i0 + (int)threadIdx.x < p.n_q ? visible_len(R, b, i0 + threadIdx.x) : 0;
    __syncthreads();
    int Lwg = 0;
#pragma unroll
    for (int q = 0; q < QB; ++q) Lwg = max(Lwg, s_L[q]);
    // this wave's queries: i0 + QW wv + q, visible lengths Lq[q]
    const int iw = i0 + QW * wv;
    int Lq[QW];
#pragma unroll
    for (int q = 0; q < QW; ++q) Lq[q] = s_L[QW * wv + q];
    const int nch = (Lwg + CK - 1) / CK;

    if (!SEL && a.fill_invisible) {
        // -inf for the positions past the computed chunks, issued first so that the stores
        // drain while the chunks are computed; 16-byte stores where the rows allow it
        const int start = min(nch * CK, p.n_kv);
        const bool vec = ((a.row_stride & 3) == 0) && (((uintptr_t)a.scores & 15) == 0);
        const int head = vec ? min(p.n_kv, (start + 3) & ~3) : p.n_kv;
        const int body = vec ? head + ((p.n_kv - head) & ~3) : p.n_kv;
        const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        for (int q = 0; q < QW; ++q) {
            const int qi = iw + q;
            if (qi >= p.n_q) break;
            float* row = a.scores + (int64_t)(b * p.n_q + qi) * a.row_stride;
            for (int j = start + lane; j < head; j += 64) row[j] = -INFINITY;
            for (int j = head + 4 * lane; j < body; j += 256) *reinterpret_cast<float4*>(row + j) = ninf;
            for (int j = body + lane; j < p.n_kv; j += 64) row[j] = -INFINITY;
        }
    }

    // SEL: candidate lists of this wave's queries (keys, then positions, cap entries each)
    // and the per-lane state of the query of this lane's group: list length and threshold
    uint32_t* slot_base = SEL ? sel.buf + (size_t)blockIdx.x * QB * 2 * sel.cap : nullptr;
    auto row_keys = [&](int q) { return slot_base + (size_t)(QW * wv + q) * 2 * sel.cap; };
    uint32_t cnt[NZ], tau[NZ];
    float tauf[NZ];  // sel_floor(tau)
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
        cnt[z] = 0;
        tau[z] = 0;
        tauf[z] = -INFINITY;
    }

    if (nch > 0) {
        // A fragments (rows 16 m + lane%16: query m / TPQ, head 16 (m % TPQ) + lane%16) and the
        // head weights of the accumulator rows (16 m + 4 (lane/16) + e)
        bf16x8 av[MT][KSTEPS];
        float wvv[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int qi = iw + m / TPQ, h = 16 * (m % TPQ) + l15;
            const bool ok = qi < p.n_q;
            const uint16_t* qp = static_cast<const uint16_t*>(a.q.data) + (ok ? (b * a.q.s0 + qi * a.q.s1 + h * a.q.s2) : 0);
#pragma unroll
            for (int s2 = 0; s2 < KSTEPS; ++s2)
                av[m][s2] = __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const uint4*>(qp + 32 * s2 + 8 * g) : make_uint4(0, 0, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wvv[m][e] = ok ? static_cast<const float*>(a.w.data)[b * a.w.s0 + qi * a.w.s1 + 16 * (m % TPQ) + 4 * g + e] : 0.f;
        }
        // a query row with a non-finite index-query element scores NaN on every visible key
        // (the plain-max ReLU alone could turn a negative NaN dot product into 0)
        bool qbad[QW];
#pragma unroll
        for (int q = 0; q < QW; ++q) qbad[q] = false;
        if (SEL || a.fix_nonfinite) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                bool bad = false;
#pragma unroll
                for (int s2 = 0; s2 < KSTEPS; ++s2) {
                    const uint4 u = __builtin_bit_cast(uint4, av[m][s2]);
                    bad |= bf16x2_nonfinite(u.x) | bf16x2_nonfinite(u.y) | bf16x2_nonfinite(u.z) | bf16x2_nonfinite(u.w);
                }
                if constexpr (SEL) {
                    int Lm = 0;
#pragma unroll
                    for (int q = 0; q < QW; ++q)
                        if (q == m / TPQ) Lm = Lq[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) bad |= !isfinite(wvv[m][e]);
                    bad_input |= bad && Lm > 0;
                } else {
                    if (__ballot(bad) != 0) qbad[m / TPQ] = true;
                }
            }
        }
        const uint32_t kstride = (uint32_t)(a.k.s1 * (KE4M3 ? 1 : 2));
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(static_cast<const uint8_t*>(a.k.data) + b * a.k.s0 * (KE4M3 ? 1 : 2)), (short)0,
            (int)((uint32_t)Lwg * kstride), 0x00020000);
        uint4 stage[PPT];
        auto fetch = [&](int c) {
            const int tid = SEL ? opaque_tid() : (int)threadIdx.x;
#pragma unroll
            for (int e = 0; e < PPT; ++e) {
                const int u = tid + 256 * e;
                const int r = u / PPR, col = u % PPR;
                const int j = c * CK + r;
                const uint32_t off = j < Lwg ? (uint32_t)j * kstride + 16u * col : 0x80000000u;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
                stage[e] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        };
        auto commit = [&](int buf) {
            const int tid = SEL ? opaque_tid() : (int)threadIdx.x;
#pragma unroll
            for (int e = 0; e < PPT; ++e) {
                const int u = tid + 256 * e;
                const int r = u / PPR, col = u % PPR;
                uint8_t* dst = &kbuf[buf][r * KP + (KE4M3 ? 32 : 16) * col];
                if constexpr (SEL) {  // keys past Lwg were loaded as zeros
                    if constexpr (KE4M3)
                        bad_input |= e4m3x4_nan(stage[e].x) | e4m3x4_nan(stage[e].y) | e4m3x4_nan(stage[e].z) |
                                     e4m3x4_nan(stage[e].w);
                    else
                        bad_input |= bf16x2_nonfinite(stage[e].x) | bf16x2_nonfinite(stage[e].y) |
                                     bf16x2_nonfinite(stage[e].z) | bf16x2_nonfinite(stage[e].w);
                }
                if constexpr (KE4M3) {
                    const uint32_t w4[4] = {stage[e].x, stage[e].y, stage[e].z, stage[e].w};
                    uint32_t o[8];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[k], 1.0f, false);
                        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[k], 1.0f, true);
                        o[2 * k] = __builtin_bit_cast(uint32_t, lo);
                        o[2 * k + 1] = __builtin_bit_cast(uint32_t, hi);
                    }
                    reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
                    reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
                } else {
                    *reinterpret_cast<uint4*>(dst) = stage[e];
                }
            }
        };
        // scores of this wave: lane group g stores query g (and g + 4 when QW = 8)
        float* srow[NZ];
        int Ls[NZ];
        bool qok[NZ];
#pragma unroll
        for (int z = 0; z < NZ; ++z) {
            const int q = g + 4 * z;
            const int qi = iw + q;
            qok[z] = q < QW && qi < p.n_q;
            srow[z] = SEL ? nullptr : a.scores + (int64_t)(b * p.n_q + (qok[z] ? qi : 0)) * a.row_stride;
            int Lz = 0;
#pragma unroll
            for (int qq = 0; qq < QW; ++qq)
                if (qq == q) Lz = Lq[qq];
            Ls[z] = qok[z] ? Lz : 0;
        }
        fetch(0);
        commit(0);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            const int buf = c & 1;
            if (c + 1 < nch) fetch(c + 1);
            const uint8_t* kb = kbuf[buf] + l15 * KP + 16 * g;
            // Software pipeline over the chunk's 16-key tiles: a query's accumulators are
            // reduced (ReLU, weights, head sum) and then refilled by the next tile's MFMAs, so
            // the epilogue's vector work sits among matrix instructions that do not depend on
            // it (no extra accumulator or B-fragment registers).
            f32x4 acc[MT];
            bf16x8 bv[KSTEPS];
            auto load_b = [&](int nt) {
#pragma unroll
                for (int s2 = 0; s2 < KSTEPS; ++s2)
                    bv[s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + nt * 16 * KP + 64 * s2));
            };
            auto mfma_tiles = [&](int m0, int m1) {  // M-tiles [m0, m1) of the tile in bv
#pragma unroll
                for (int s2 = 0; s2 < KSTEPS; ++s2)
#pragma unroll
                    for (int m = m0; m < m1; ++m)
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][s2], bv[s2], s2 == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[m],
                                                                       0, 0, 0);
            };
            auto reduce_q = [&](int q) {
                // four partial sums (short dependency chains); the ReLU is the
                // one-instruction integer max (non-finite inputs are handled apart)
                float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = q * TPQ; m < (q + 1) * TPQ; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] = fmaf(wvv[m][e], relu_finite(acc[m][e]), t[e]);
                return xsum32(xsum16((t[0] + t[1]) + (t[2] + t[3])));
            };
            auto emit = [&](int nt, const float (&sc)[QW]) {
                const int j = c * CK + nt * 16 + l15;
#pragma unroll
                for (int z = 0; z < NZ; ++z) {
                    float v = 0.f;
#pragma unroll
                    for (int q = 0; q < QW; ++q)
                        if (q == g + 4 * z) v = sc[q];
                    const bool vis = j < Ls[z];
                    if constexpr (SEL) {
                        // append above-threshold scores in position order (lanes of a group
                        // hold consecutive keys)
                        const bool pass = vis && v >= tauf[z];
                        const uint64_t mk = __ballot(pass);
                        const uint32_t gm = (uint32_t)(mk >> (16 * g)) & 0xffffu;
                        if (pass) {
                            const uint32_t key = sel_key(v);
                            const uint32_t slot = cnt[z] + (uint32_t)__builtin_popcount(gm & ((1u << l15) - 1u));
                            uint32_t* lk = row_keys(g + 4 * z);
                            lk[slot] = key;
                            lk[sel.cap + slot] = (uint32_t)j;
                            if (c > 0) {  // the row's bins exist from the second chunk on
                                const int r = QW * wv + g + 4 * z;
                                atomicAdd(&s_rh[r][sel_bin<NBR>(v, s_rp[r][0], (int)s_rp[r][1])], 1u);
                            }
                        }
                        cnt[z] += (uint32_t)__builtin_popcount(gm);
                    } else {
                        bool qb = false;
#pragma unroll
                        for (int q = 0; q < QW; ++q)
                            if (q == g + 4 * z) qb = qbad[q];
                        if (qok[z] && j < p.n_kv && (vis || a.fill_invisible)) srow[z][j] = vis ? (qb ? __builtin_nanf("") : v) : -INFINITY;
                    }
                }
            };
            // Rotation per tile nt: reduce query 0 of nt beside the MFMAs of nt's last query,
            // then (B fragment of nt + 1) for q >= 1 reduce query q of nt beside the MFMAs of
            // nt + 1 for query q - 1, then store or list the scores.  (Pinning the MFMA / vector
            // interleave with scheduling-group barriers measured no faster.)
            constexpr int NT = CK / 16;
            load_b(0);
            mfma_tiles(0, (QW - 1) * TPQ);
#pragma unroll 1
            for (int nt = 0; nt < NT; ++nt) {
                float sc[QW];
                sc[0] = reduce_q(0);
                mfma_tiles((QW - 1) * TPQ, QW * TPQ);
                const bool more = nt + 1 < NT;
                if (more) load_b(nt + 1);
#pragma unroll
                for (int q = 1; q < QW; ++q) {
                    sc[q] = reduce_q(q);
                    if (more) mfma_tiles((q - 1) * TPQ, q * TPQ);
                }
                emit(nt, sc);
            }
            if (c + 1 < nch) commit(buf ^ 1);
            __syncthreads();
            if constexpr (SEL) {
                // per row of this wave: bins after the first chunk, a higher threshold from
                // the histogram, and dead entries dropped when the next chunk could overflow
                if (c + 1 < nch) {
                    const int ln = opaque_tid() & 63;
                    if (c == 0) {
                        // bins from each row's first chunk: every visible key of it is listed (n <= 128)
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
                        for (int q = 0; q < QW; ++q) {
                            const int z = q >> 2, gq = q & 3, r = QW * wv + q;
                            const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)cnt[z], 16 * gq);
                            const uint32_t* keys = row_keys(q);
                            const uint32_t k0 = ln < (int)n ? keys[ln] : 0xffffffffu;
                            const uint32_t k1 = ln + 64 < (int)n ? keys[ln + 64] : 0xffffffffu;
                            const uint32_t lo = wave_min(min(k0, k1));
                            const uint32_t hi = wave_max(max(ln < (int)n ? k0 : 0u, ln + 64 < (int)n ? k1 : 0u));
                            uint32_t wb = 127u << 23;
                            int j0 = 0;
                            if (n) sel_bins<NBR>(lo, hi, wb, j0);
                            if (ln == 0) {
                                s_rp[r][0] = wb;
                                s_rp[r][1] = (uint32_t)j0;
                            }
                            if (4 * ln < NBR) *reinterpret_cast<uint4*>(&s_rh[r][4 * ln]) = make_uint4(0u, 0u, 0u, 0u);
                            if (ln < (int)n) atomicAdd(&s_rh[r][sel_bin<NBR>(sel_val(k0), wb, j0)], 1u);
                            if (ln + 64 < (int)n) atomicAdd(&s_rh[r][sel_bin<NBR>(sel_val(k1), wb, j0)], 1u);
                        }
                        wait_lgkmcnt0();
                    }
                    // every other chunk, and before a cut: a higher threshold from each row's
                    // histogram; with four or eight rows per wave all rows at once (lane group g
                    // holds row g + 4 z), with two (and many more bins) one row after the other
                    if constexpr (QW >= 4) {
#pragma unroll
                        for (int z = 0; z < NZ; ++z) {
                            const int r = QW * wv + g + 4 * z;
                            const bool full = cnt[z] + CK > (uint32_t)sel.cap;
                            const bool upd = cnt[z] >= (uint32_t)K && ((c & 1) == 0 || full);
                            if (__ballot(upd) != 0) {
                                const int bk = sel_find_bin_rows<NBR>(s_rh[r], (uint32_t)K, l15);
                                if (upd && bk >= 1) tau[z] = max(tau[z], bin_lowest(bk, s_rp[r][0], (int)s_rp[r][1]) - 1u);
                            }
                            tauf[z] = sel_floor(tau[z]);
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < QW; ++q) {
                            const int r = QW * wv + q;
                            const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)cnt[0], 16 * q);
                            const bool full = n + CK > (uint32_t)sel.cap;
                            if (n >= (uint32_t)K && ((c & 1) == 0 || full)) {
                                int bk;
                                uint32_t above;
                                sel_find_bin<NBR>(s_rh[r], (uint32_t)K, ln, bk, above);
                                if (bk >= 1 && g == q) tau[0] = max(tau[0], bin_lowest(bk, s_rp[r][0], (int)s_rp[r][1]) - 1u);
                            }
                        }
                        tauf[0] = sel_floor(tau[0]);
                    }
                    // rows whose list could overflow at the next chunk: drop the entries at or
                    // below the threshold, or cut to the exact top k when that frees too little
#pragma unroll
                    for (int q = 0; q < QW; ++q) {
                        const int z = q >> 2, gq = q & 3, r = QW * wv + q;
                        uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)cnt[z], 16 * gq);
                        if (n + CK <= (uint32_t)sel.cap) continue;
                        uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)tau[z], 16 * gq);
                        uint32_t* keys = row_keys(q);
                        int32_t* pos = reinterpret_cast<int32_t*>(keys + sel.cap);
                        const uint32_t wb = s_rp[r][0];
                        const int j0 = (int)s_rp[r][1];
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's appends have landed
                        n = sel_compact(keys, pos, (int)n, t, 0u, keys, pos, ln);  // keys > t
                        const int bt = sel_bin<NBR>(sel_val(t + 1u), wb, j0);  // the bins below hold keys <= t
                        for (int e = ln; e < bt; e += 64) s_rh[r][e] = 0u;
                        if (n + CK > (uint32_t)sel.cap) {
                            // keys far outside the bins: cut to the exact top k, new bins from there
                            uint32_t T, need_eq, hi;
                            sel_threshold(keys, (int)n, (uint32_t)K, &s_sel[wv], ln, T, need_eq, hi);
                            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                            n = sel_compact(keys, pos, (int)n, T, need_eq, keys, pos, ln);
                            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                            uint32_t wb2;
                            int j02;
                            sel_bins<NBR>(T, hi, wb2, j02);
                            if (ln == 0) {
                                s_rp[r][0] = wb2;
                                s_rp[r][1] = (uint32_t)j02;
                            }
                            for (int e = ln; e < NBR; e += 64) s_rh[r][e] = 0u;
                            for (int e = ln; e < (int)n; e += 64) atomicAdd(&s_rh[r][sel_bin<NBR>(sel_val(keys[e]), wb2, j02)], 1u);
                            t = T > 0u ? T - 1u : 0u;
                        }
                        wait_lgkmcnt0();
                        if (g == gq) {
                            cnt[z] = n;
                            tau[z] = t;
                            tauf[z] = sel_floor(t);
                        }
                    }
                }
            }
        }
    }
    if constexpr (SEL) {
        // the selection of each of this wave's rows, in ascending position, -1 padded: the
        // k-th key from the histogram's bin and digits of it, then one ordered pass
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int ln = opaque_tid() & 63;
        const bool binned = nch > 1;  // the bins were made after the first of several chunks
#pragma unroll
        for (int q = 0; q < QW; ++q) {
            const int qi = iw + q;
            if (qi >= p.n_q) break;
            const int z = q >> 2, gq = q & 3, r = QW * wv + q;
            int32_t* out = sel.idx + ((int64_t)b * p.n_q + qi) * K;
            const uint32_t n = Lq[q] > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)cnt[z], 16 * gq) : 0u;
            uint32_t* keys = row_keys(q);
            int32_t* pos = reinterpret_cast<int32_t*>(keys + sel.cap);
            if (n <= (uint32_t)K) {
                for (int e = ln; e < K; e += 64) out[e] = e < (int)n ? pos[e] : -1;
            } else {
                uint32_t T, need_eq;
                int bk = 0;
                uint32_t above = 0;
                if (binned) sel_find_bin<NBR>(s_rh[r], (uint32_t)K, ln, bk, above);
                if (binned && bk >= 1 && bk < NBR - 1) {
                    const uint32_t wb = s_rp[r][0];
                    const int j0 = (int)s_rp[r][1];
                    const uint32_t lo = bin_lowest(bk, wb, j0), top = bin_lowest(bk + 1, wb, j0) - 1u;
                    const uint32_t span = top - lo;
                    const int bits = span == 0 ? 0 : 32 - __clz((int)span);
                    sel_refine(keys, (int)n, lo, top, bits, 0u, s_rh[r][bk], (uint32_t)K - above, &s_sel[wv], ln, T,
                               need_eq);
                } else {
                    uint32_t hi;
                    sel_threshold(keys, (int)n, (uint32_t)K, &s_sel[wv], ln, T, need_eq, hi);
                }
                sel_compact(keys, pos, (int)n, T, need_eq, nullptr, out, ln);
            }
        }
    }
    }  // rounds
    if constexpr (SEL) {
        if (__ballot(bad_input) != 0 && (threadIdx.x & 63) == 0) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
    }
}

// ----------------------------------------------------- matrix-core path, LDS key chunks
// The workgroup streams its key range through LDS in chunks of 128 keys, double-buffered:
// all 256 threads fetch the next chunk with 16-byte loads while the waves multiply the
// current one, so the memory wait is paid once per chunk.  Prefill: wave w owns query
// group qb*4 + w (all four 16-row M-tiles) and the four groups share every chunk.
// Decode (64 index heads, one query per group): wave w owns heads 16w..16w+15 of the
// workgroup's query; the four 16-head partial sums of each position meet in LDS and are
// added in the fixed order 0+1+2+3.  Key rows are padded in LDS (8 bytes for e4m3, 16 for
// bf16) so the 16 rows a fragment load touches fall in different banks.
constexpr int kCK = 128;  // keys per LDS chunk

template <int KSTEPS, bool KE4M3, int H, bool DECODE, bool FAST_RELU>
__global__ void __launch_bounds__(256) indexer_mfma3(IndexerArgs a, int n_groups, int n_qblk, int n_rng, int rng_len) {
    constexpr int D = 32 * KSTEPS;
    constexpr int RB = D * (KE4M3 ? 1 : 2);      // key row bytes
    constexpr int RBP = RB + (KE4M3 ? 8 : 16);    // padded LDS row pitch (keeps fragment alignment)
    constexpr int U16 = kCK * RB / 16;            // 16-byte pieces per chunk
    constexpr int PPT = U16 / 256;                // pieces per thread
    constexpr int QPG = 64 / H;
    constexpr int MW = DECODE ? 1 : kMT;          // M-tiles per wave
    static_assert(!DECODE || H == 64, "decode layout splits the 64 index heads of one query");
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kCK * RBP];
    __shared__ float red[DECODE ? 4 * kCK : 1];

    const sa_problem& p = a.p;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long wg = blockIdx.x;
    const int rng = (int)(wg % n_rng);
    const long rest = wg / n_rng;
    int b, g;
    if (DECODE) {
        g = (int)(rest % n_groups);
        b = (int)(rest / n_groups);
    } else {
        const int qb = n_qblk - 1 - (int)(rest % n_qblk);  // longest causal histories first
        b = (int)(rest / n_qblk);
        g = qb * 4 + wv;
    }
    const int j_begin = rng * rng_len;
    const int j_end = min(j_begin + rng_len, p.n_kv);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    // visible lengths: lane q of a wave holds query q of its group
    const int i0 = g * QPG;
    int Lq = 0;
    if (g < n_groups && lane < QPG && i0 + lane < p.n_q) Lq = visible_len(R, b, i0 + lane);
    int Lw = Lq;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Lw = max(Lw, __shfl_xor(Lw, o));
    // workgroup-wide end of the keys worth computing
    __shared__ int s_L[4];
    if (lane == 0) s_L[wv] = Lw;
    __syncthreads();
    const int Lwg = max(max(s_L[0], s_L[1]), max(s_L[2], s_L[3]));
    const int j_comp_end = min(j_end, Lwg);
    const bool wave_live = g < n_groups;

    if (j_begin < j_comp_end) {
        // this wave's A fragments and head weights
        bf16x8 av[MW][KSTEPS];
        float wvv[MW][4];
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int mt = DECODE ? wv : m;
            const int r = 16 * mt + (lane & 15);
            const int qi = i0 + r / H, h = r % H;
            const bool ok = wave_live && qi < p.n_q;
            const uint16_t* qb = static_cast<const uint16_t*>(a.q.data) + (ok ? (b * a.q.s0 + qi * a.q.s1 + h * a.q.s2) : 0);
#pragma unroll
            for (int s2 = 0; s2 < KSTEPS; ++s2) {
                uint4 u = ok ? *reinterpret_cast<const uint4*>(qb + 32 * s2 + 8 * (lane >> 4)) : make_uint4(0, 0, 0, 0);
                av[m][s2] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * mt + 4 * (lane >> 4) + e;
                const int q2 = i0 + rr / H, h2 = rr % H;
                wvv[m][e] = (wave_live && q2 < p.n_q) ? static_cast<const float*>(a.w.data)[b * a.w.s0 + q2 * a.w.s1 + h2] : 0.f;
            }
        }
        const uint32_t kstride_bytes = (uint32_t)(a.k.s1 * (KE4M3 ? 1 : 2));
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(static_cast<const uint8_t*>(a.k.data) + b * a.k.s0 * (KE4M3 ? 1 : 2)), (short)0,
            (int)((uint32_t)j_comp_end * kstride_bytes), 0x00020000);
        const int nrows = wave_live ? min(QPG, p.n_q - i0) : 0;
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            a.scores + (int64_t)(b * p.n_q + (wave_live ? i0 : 0)) * a.row_stride, (short)0,
            (int)((uint32_t)nrows * (uint32_t)a.row_stride * 4u), 0x00020000);

        uint4 stage[PPT];
        auto fetch = [&](int c) {
#pragma unroll
            for (int e = 0; e < PPT; ++e) {
                const int u = threadIdx.x + 256 * e;
                const int r = u / (RB / 16), col = u % (RB / 16);
                const int j = j_begin + c * kCK + r;
                const uint32_t off = j < j_comp_end ? (uint32_t)j * kstride_bytes + 16u * col : 0x80000000u;
                auto v = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
                stage[e] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        };
        auto commit = [&](int buf) {
#pragma unroll
            for (int e = 0; e < PPT; ++e) {
                const int u = threadIdx.x + 256 * e;
                const int r = u / (RB / 16), col = u % (RB / 16);
                if constexpr (RBP % 16 == 0) {
                    *reinterpret_cast<uint4*>(&kbuf[buf][r * RBP + 16 * col]) = stage[e];
                } else {
                    *reinterpret_cast<uint2*>(&kbuf[buf][r * RBP + 16 * col]) = make_uint2(stage[e].x, stage[e].y);
                    *reinterpret_cast<uint2*>(&kbuf[buf][r * RBP + 16 * col + 8]) = make_uint2(stage[e].z, stage[e].w);
                }
            }
        };
        const int nch = (j_comp_end - j_begin + kCK - 1) / kCK;
        fetch(0);
        commit(0);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            const int buf = c & 1;
            if (c + 1 < nch) fetch(c + 1);
            const int cbase = j_begin + c * kCK;
            const int ntile = min(kCK, j_comp_end - cbase + 15) / 16;
            for (int tI = 0; tI < ntile; ++tI) {
                const int jl = 16 * tI + (lane & 15);
                const int j = cbase + jl;
                bf16x8 bv[KSTEPS];
                const uint8_t* kr = &kbuf[buf][jl * RBP + 8 * (lane >> 4) * (KE4M3 ? 1 : 2)];
#pragma unroll
                for (int s2 = 0; s2 < KSTEPS; ++s2) {
                    if constexpr (KE4M3) {
                        const uint2 u = *reinterpret_cast<const uint2*>(kr + 32 * s2);
                        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.x, 1.0f, false);
                        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.x, 1.0f, true);
                        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.y, 1.0f, false);
                        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.y, 1.0f, true);
                        bv[s2] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                    } else {
                        bv[s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + 64 * s2));
                    }
                }
                f32x4 acc[MW];
#pragma unroll
                for (int m = 0; m < MW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < KSTEPS; ++s2)
#pragma unroll
                    for (int m = 0; m < MW; ++m)
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][s2], bv[s2], acc[m], 0, 0, 0);
                float part[MW];
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    float t = 0.f, chk = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float z = acc[m][e];
                        t = fmaf(wvv[m][e], relu_finite(z), t);
                        if (!FAST_RELU) chk = fmaf(z, 0.f, chk);  // NaN for a non-finite dot product
                    }
                    part[m] = FAST_RELU ? t : t + chk;
                }
                if constexpr (DECODE) {
                    float v = part[0];
                    v = xsum32(xsum16(v));
                    if (lane < 16) red[wv * kCK + jl] = v;
                } else if constexpr (H >= 16) {
                    constexpr int tpq = H / 16;
#pragma unroll
                    for (int q = 0; q < QPG; ++q) {
                        float v = 0.f;
#pragma unroll
                        for (int t = 0; t < tpq; ++t) v += part[q * tpq + t];
                        v = xsum32(xsum16(v));
                        const int Lh = __shfl(Lq, q);
                        const bool vis = j < Lh;
                        const bool wr = wave_live && lane < 16 && i0 + q < p.n_q && j < j_end && (vis || a.fill_invisible);
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, vis ? v : -INFINITY), srs,
                                                              wr ? (uint32_t)(q * a.row_stride + j) * 4u : 0x80000000u, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt) {
                        float v = part[mt];
                        int qloc;
                        if constexpr (H == 8) {
                            v = xsum16(v);
                            qloc = 2 * mt + (lane >> 5);
                        } else {
                            qloc = 4 * mt + (lane >> 4);
                        }
                        const int Lh = __shfl(Lq, qloc);
                        const bool writer = (H == 8) ? ((lane & 16) == 0) : true;
                        const bool vis = j < Lh;
                        const bool wr = wave_live && writer && i0 + qloc < p.n_q && j < j_end && (vis || a.fill_invisible);
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, vis ? v : -INFINITY), srs,
                                                              wr ? (uint32_t)(qloc * a.row_stride + j) * 4u : 0x80000000u, 0, 0);
                    }
                }
            }
            if constexpr (DECODE) {
                __syncthreads();
                if (threadIdx.x < kCK) {
                    const int j = cbase + threadIdx.x;
                    const float v = ((red[threadIdx.x] + red[kCK + threadIdx.x]) + red[2 * kCK + threadIdx.x]) +
                                    red[3 * kCK + threadIdx.x];
                    const int L0 = __shfl(Lq, 0);  // lane 0 of each wave holds the query's length
                    const bool vis = j < L0;
                    const bool wr = (int)threadIdx.x < 16 * ntile && j < j_end && (vis || a.fill_invisible) && i0 < p.n_q;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, vis ? v : -INFINITY), srs, wr ? (uint32_t)j * 4u : 0x80000000u, 0, 0);
                }
            }
            if (c + 1 < nch) commit(buf ^ 1);
            __syncthreads();
        }
    }
    if (a.fill_invisible && wave_live) {
        // positions past the computed chunks (or the whole range when nothing was computed)
        const int start = j_begin < j_comp_end ? j_begin + ((j_comp_end - j_begin + 15) / 16) * 16 : j_begin;
        const int qs = DECODE ? (wv == 0 ? 0 : QPG) : 0;  // in decode only wave 0 fills
        for (int q = qs; q < QPG; ++q) {
            const int qi = i0 + q;
            if (qi >= p.n_q) break;
            float* row = a.scores + (int64_t)(b * p.n_q + qi) * a.row_stride;
            for (int j = start + lane; j < j_end; j += 64) row[j] = -INFINITY;
        }
    }
}

// Non-finite check of the index inputs a query row can see (bf16 index queries with bf16
// or e4m3 index keys, d_idx a multiple of 16): valid query rows of q_idx and w, and index
// keys below the longest visible history of each batch.  16-byte chunks; bf16 values are
// non-finite when their exponent bits are all ones, e4m3 bytes when their low seven bits
// are (0x7f / 0xff, the format's only non-finite codes).
__global__ void __launch_bounds__(256) index_finite_check(IndexerArgs a) {
    const sa_problem& p = a.p;
    const int b = blockIdx.y;
    int kl = p.kv_len ? p.kv_len[b] : p.n_kv;
    kl = kl < 0 ? 0 : (kl > p.n_kv ? p.n_kv : kl);
    const long qp0 = p.q_pos0 ? p.q_pos0[b] : 0;
    if (qp0 >= kl) return;  // no valid query row in this batch
    const int Lb = p.causal ? (int)min((long)kl, qp0 + p.n_q) : kl;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    bool bad = false;
    const long tid = (long)blockIdx.x * 256 + threadIdx.x, nth = (long)gridDim.x * 256;
    const bool e4 = a.k.dtype == SA_FP8_E4M3;
    const int kch = p.d_idx * (e4 ? 1 : 2) / 16;  // 16-byte chunks per key row
    const uint8_t* kb = static_cast<const uint8_t*>(a.k.data) + b * a.k.s0 * (e4 ? 1 : 2);
    for (long e = tid; e < (long)Lb * kch; e += nth) {
        const long j = e / kch;
        const int c = (int)(e % kch);
        const uint4 u = *reinterpret_cast<const uint4*>(kb + j * a.k.s1 * (e4 ? 1 : 2) + 16 * c);
        if (e4) bad |= e4m3x4_nan(u.x) | e4m3x4_nan(u.y) | e4m3x4_nan(u.z) | e4m3x4_nan(u.w);
        else bad |= bf16x2_nonfinite(u.x) | bf16x2_nonfinite(u.y) | bf16x2_nonfinite(u.z) | bf16x2_nonfinite(u.w);
    }
    const int qch = p.d_idx / 8;  // 16-byte chunks per index-head vector
    const long per_row = (long)p.Hidx * qch;
    for (long e = tid; e < (long)p.n_q * per_row; e += nth) {
        const int i = (int)(e / per_row);
        if (visible_len(R, b, i) == 0) continue;
        const int h = (int)((e % per_row) / qch), c = (int)(e % qch);
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q.data) + b * a.q.s0 +
                                                         (int64_t)i * a.q.s1 + h * a.q.s2 + 8 * c);
        bad |= bf16x2_nonfinite(u.x) | bf16x2_nonfinite(u.y) | bf16x2_nonfinite(u.z) | bf16x2_nonfinite(u.w);
    }
    for (long e = tid; e < (long)p.n_q * p.Hidx; e += nth) {
        const int i = (int)(e / p.Hidx), h = (int)(e % p.Hidx);
        if (visible_len(R, b, i) == 0) continue;
        if (!isfinite(static_cast<const float*>(a.w.data)[b * a.w.s0 + (int64_t)i * a.w.s1 + h])) bad = true;
    }
    if (bad) atomicOr(&a.status->flags, 1u << SA_ERR_NONFINITE);
}

// Keys with a non-finite index-key element score NaN for every query row that sees them
// (the plain-max ReLU alone could turn a negative NaN dot product into 0).  Runs after the
// score kernel; each thread checks one 16-byte chunk of one key row.
__global__ void __launch_bounds__(256) index_key_fix(IndexerArgs a) {
    const sa_problem& p = a.p;
    const int b = blockIdx.y;
    int kl = p.kv_len ? p.kv_len[b] : p.n_kv;
    kl = kl < 0 ? 0 : (kl > p.n_kv ? p.n_kv : kl);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal, a.row_len};
    const bool e4 = a.k.dtype == SA_FP8_E4M3;
    const int kch = p.d_idx * (e4 ? 1 : 2) / 16;
    const uint8_t* kb = static_cast<const uint8_t*>(a.k.data) + b * a.k.s0 * (e4 ? 1 : 2);
    for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < (long)kl * kch; e += (long)gridDim.x * 256) {
        const long j = e / kch;
        const int c = (int)(e % kch);
        const uint4 u = *reinterpret_cast<const uint4*>(kb + j * a.k.s1 * (e4 ? 1 : 2) + 16 * c);
        const bool bad = e4 ? (e4m3x4_nan(u.x) | e4m3x4_nan(u.y) | e4m3x4_nan(u.z) | e4m3x4_nan(u.w))
                            : (bf16x2_nonfinite(u.x) | bf16x2_nonfinite(u.y) | bf16x2_nonfinite(u.z) | bf16x2_nonfinite(u.w));
        if (!bad) continue;
        for (int i = 0; i < p.n_q; ++i)
            if (j < visible_len(R, b, i)) a.scores[(int64_t)(b * p.n_q + i) * a.row_stride + j] = __builtin_nanf("");
    }
}

}  // namespace

// The fused score + select runs on the many-row prefill layout: bf16 index queries, bf16 or
// e4m3 index keys, 16 / 32 / 64 index heads of width 64 or 128, and enough blocks of query
// rows to fill the chip.  A candidate list holds min(4k + 512, n_kv + 128) entries: room
// for the k(1 + ln(L / k)) or so keys a row of L positions appends when its scores come in
// no particular order, so that lists are rarely cut before the end, and never less than k
// plus one chunk of keys (n_kv >= k) or the whole history (n_kv < k).
namespace {
int sel_qb(const sa_problem& p) { return 4 * 128 / p.Hidx; }
int sel_cap(const sa_problem& p) {
    const long c = std::min(4L * p.k + 512, (long)p.n_kv + 128);
    return (int)((c + 63) & ~63L);
}
long sel_slots(const sa_problem& p) {
    const long items = (long)p.B * ((p.n_q + sel_qb(p) - 1) / sel_qb(p));
    return std::min(items, (long)kSelSlots);
}
}  // namespace

bool select_fused_shape_ok(const sa_problem& p) {
    const int H = p.Hidx, D = p.d_idx;
    if (!(H == 16 || H == 32 || H == 64) || !(D == 64 || D == 128)) return false;
    const long rows = (long)p.B * p.n_q;
    if (rows < 512 || (H == 64 && rows < 1024)) return false;  // the few-row and decode layouts
    const long n_qb = (p.n_q + sel_qb(p) - 1) / sel_qb(p);
    return (long)p.B * n_qb >= 512;
}

bool select_fused_ok(const sa_problem& p, int q_dtype, int k_dtype) {
    return q_dtype == SA_BF16 && (k_dtype == SA_BF16 || k_dtype == SA_FP8_E4M3) && select_fused_shape_ok(p);
}

size_t select_fused_bytes(const sa_problem& p) {
    return (size_t)sel_slots(p) * sel_qb(p) * 2 * (size_t)sel_cap(p) * sizeof(uint32_t);
}

hipError_t launch_select_fused(const IndexerArgs& a, int32_t* idx, void* buf, hipStream_t s) {
    const sa_problem& p = a.p;
    if (!select_fused_ok(p, a.q.dtype, a.k.dtype) || !a.status) return hipErrorInvalidValue;
    SelectArgs sel;
    sel.buf = static_cast<uint32_t*>(buf);
    sel.cap = sel_cap(p);
    sel.idx = idx;
    const int QB = sel_qb(p);
    const int n_qb = (p.n_q + QB - 1) / QB;
    const dim3 grid((unsigned)sel_slots(p)), block(256);
    const bool e4 = a.k.dtype == SA_FP8_E4M3;
    IndexerArgs af = a;
    af.fill_invisible = 0;
    af.fix_nonfinite = 0;
#define SA_SEL(KS, E4, HH)                                                                                    \
    if (p.Hidx == HH) {                                                                                       \
        hipLaunchKernelGGL((indexer_pf<KS, E4, HH, true>), grid, block, 0, s, af, n_qb, sel);                 \
        return hipGetLastError();                                                                             \
    }
#define SA_SEL_H(KS, E4) do { SA_SEL(KS, E4, 16) SA_SEL(KS, E4, 32) SA_SEL(KS, E4, 64) } while (0)
    if (p.d_idx == 64) { if (e4) SA_SEL_H(2, true); else SA_SEL_H(2, false); }
    else { if (e4) SA_SEL_H(4, true); else SA_SEL_H(4, false); }
#undef SA_SEL_H
#undef SA_SEL
    return hipErrorInvalidValue;
}

bool indexer_dec_path(const IndexerArgs& a) {
    const sa_problem& p = a.p;
    const int H = p.Hidx, D = p.d_idx;
    const bool mfma_ok = a.nrows == 0 && a.q.dtype == SA_BF16 && (a.k.dtype == SA_BF16 || a.k.dtype == SA_FP8_E4M3) &&
                         (H == 4 || H == 8 || H == 16 || H == 32 || H == 64) &&
                         (D == 32 || D == 64 || D == 128);
    return mfma_ok && (long)p.B * p.n_q < 512 && H >= 16 && D >= 64;
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
    const sa_problem& p = a.p;
    if (a.hist0 && !indexer_dec_path(a)) return hipErrorInvalidValue;  // only indexer_dec fills it
    const int H = p.Hidx, D = p.d_idx;
    const bool mfma_ok = a.nrows == 0 && a.q.dtype == SA_BF16 && (a.k.dtype == SA_BF16 || a.k.dtype == SA_FP8_E4M3) &&
                         (H == 4 || H == 8 || H == 16 || H == 32 || H == 64) &&
                         (D == 32 || D == 64 || D == 128);
    if (mfma_ok) {
        const int QPG = 64 / H;
        const int n_groups = (p.n_q + QPG - 1) / QPG;
        // decode layout (the four waves split one query's 64 index heads) for few query groups
        const bool decode = H == 64 && (long)p.B * n_groups < 1024;
        const bool few_rows = indexer_dec_path(a);  // indexer_dec below
        const bool fast = a.status != nullptr && !decode && !few_rows;
        if (fast) {
            const dim3 gc((unsigned)max(1L, min(512L, 65536L / p.B)), p.B);
            hipLaunchKernelGGL(index_finite_check, gc, dim3(256), 0, s, a);
        }
        // few query rows: waves split the keys of one row, keys read straight into registers
        if (few_rows) {
            const int rng_len = 1024;  // (2048 measured 3% slower on the decode workloads: a longer tail)
            const int n_rng = (p.n_kv + rng_len - 1) / rng_len;
            const dim3 gd((unsigned)((long)p.B * p.n_q * n_rng)), bd(256);
            const bool e4 = a.k.dtype == SA_FP8_E4M3;
#define SA_IDXD(KS, E4, HH)                                                                                   \
    if (H == HH) {                                                                                            \
        hipLaunchKernelGGL((indexer_dec<KS, E4, HH, false>), gd, bd, 0, s, a, n_rng, rng_len);                \
        return hipGetLastError();                                                                             \
    }
#define SA_IDXD_H(KS, E4) do { SA_IDXD(KS, E4, 16) SA_IDXD(KS, E4, 32) SA_IDXD(KS, E4, 64) } while (0)
            if (D == 64) { if (e4) SA_IDXD_H(2, true); else SA_IDXD_H(2, false); }
            else { if (e4) SA_IDXD_H(4, true); else SA_IDXD_H(4, false); }
#undef SA_IDXD_H
#undef SA_IDXD
        }
        // prefill with many query rows: one pass over the history per block of query rows
        if (!decode && H >= 16 && D >= 64) {
            const int QB = 4 * 128 / H;
            const int n_qb = (p.n_q + QB - 1) / QB;
            if ((long)p.B * n_qb >= 512) {
                const dim3 gp((unsigned)((long)p.B * n_qb)), bp(256);
                const bool e4 = a.k.dtype == SA_FP8_E4M3;
                // without the pre-pass (standalone scores): the plain-max kernel with NaN for
                // non-finite query rows, then NaN for non-finite keys
                IndexerArgs af = a;
                af.fix_nonfinite = fast ? 0 : 1;
                const dim3 gk((unsigned)max(1L, min(512L, 65536L / p.B)), p.B);
#define SA_IDXPF(KS, E4, HH)                                                                                  \
    if (H == HH) {                                                                                            \
        hipLaunchKernelGGL((indexer_pf<KS, E4, HH, false>), gp, bp, 0, s, af, n_qb, SelectArgs());            \
        if (!fast) hipLaunchKernelGGL(index_key_fix, gk, dim3(256), 0, s, af);                                \
        return hipGetLastError();                                                                             \
    }
#define SA_IDXPF_H(KS, E4) do { SA_IDXPF(KS, E4, 16) SA_IDXPF(KS, E4, 32) SA_IDXPF(KS, E4, 64) } while (0)
                if (D == 64) { if (e4) SA_IDXPF_H(2, true); else SA_IDXPF_H(2, false); }
                else { if (e4) SA_IDXPF_H(4, true); else SA_IDXPF_H(4, false); }
#undef SA_IDXPF_H
#undef SA_IDXPF
            }
        }
        const int rng_len = decode ? 2048 : 1024;
        const int n_rng = (p.n_kv + rng_len - 1) / rng_len;
        const int n_qblk = (n_groups + 3) / 4;
        const long wgs = decode ? (long)p.B * n_groups * n_rng : (long)p.B * n_qblk * n_rng;
        const bool e4 = a.k.dtype == SA_FP8_E4M3;
        const dim3 gw((unsigned)wgs), bw(256);
#define SA_IDX3(KS, E4, HH)                                                                                   \
    if (H == HH) {                                                                                            \
        if constexpr (HH == 64) {                                                                             \
            if (decode) {                                                                                     \
                hipLaunchKernelGGL((indexer_mfma3<KS, E4, HH, true, false>), gw, bw, 0, s, a, n_groups, n_qblk, n_rng, rng_len); \
                return hipGetLastError();                                                                     \
            }                                                                                                 \
        }                                                                                                     \
        if (fast) hipLaunchKernelGGL((indexer_mfma3<KS, E4, HH, false, true>), gw, bw, 0, s, a, n_groups, n_qblk, n_rng, rng_len); \
        else hipLaunchKernelGGL((indexer_mfma3<KS, E4, HH, false, false>), gw, bw, 0, s, a, n_groups, n_qblk, n_rng, rng_len);    \
    }
#define SA_IDX3_KS(KS, E4) \
    do { SA_IDX3(KS, E4, 4) SA_IDX3(KS, E4, 8) SA_IDX3(KS, E4, 16) SA_IDX3(KS, E4, 32) SA_IDX3(KS, E4, 64) } while (0)
        if (D == 32) { if (e4) SA_IDX3_KS(1, true); else SA_IDX3_KS(1, false); }
        else if (D == 64) { if (e4) SA_IDX3_KS(2, true); else SA_IDX3_KS(2, false); }
        else { if (e4) SA_IDX3_KS(4, true); else SA_IDX3_KS(4, false); }
#undef SA_IDX3_KS
#undef SA_IDX3
        return hipGetLastError();
    }
    dim3 grid(a.nrows > 0 ? a.nrows : p.B * p.n_q, (p.n_kv + 255) / 256);
    size_t shm = sizeof(float) * ((size_t)H * D + H);
    hipLaunchKernelGGL(indexer_valu, grid, dim3(256), shm, s, a);
    return hipGetLastError();
}

}  // namespace sa
