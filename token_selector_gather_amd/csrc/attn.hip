// Sparse gather attention over a selected candidate set.
//
// For query row (b,i), main head h (key/value head h / (Hq/Hkv)) and the valid entries
// j of idx[b,i,:]:  l_j = scale * <Q[b,h,i,:], K[b,hk,j,:]>, one softmax over the whole
// set (shared row maximum and exp-sum), O = sum_j p_j V[b,hk,j,:], LSE = max + ln(sum)
// ("PaperTrace 2.1.1 · Hashing and clustering", §1.1 eq. (1) and §5.1; the logit of
// "PaperTrace 2.2 · Fine-grained indexing", §3.2).  Entries that are -1, out of range or
// not visible are never read.  Split pieces of one set are merged by log-sum-exp (the
// block-mixture identity of the COBS reading note, eq. (P3)).
//
// Kernels:
//  * attn_rows_buf: bf16 MHA (one query head per key/value head, width 64/128/256).  One wave
//    per (query row, key/value head); lane groups fetch whole rows with raw buffer loads and
//    keep their own online-softmax state, merged once at the end.  Work items are laid out
//    so that each of the 8 XCDs serves a fixed subset of key/value heads, keeping that
//    subset's K/V rows in its own L2.
//  * attn_rows: the general fallback (f32, GQA groups of 2 or 4, other widths).
//  * attn_mla_lds: one latent key/value head shared by 32, 64 or 128 query heads (V = the
//    first d_v columns of K).  Gathered rows reach LDS through buffer loads that write LDS
//    directly; S^T on 16x16x32 MFMA chains, P exchanged through LDS, each wave accumulating
//    O^T for its slice of the value columns (see the kernel's own comment).
//  * attn_mla: the latent fallback for other multiples of 16 heads or a separate V tensor;
//    rows staged in LDS row-major for S^T = K Q^T and transposed for O^T += V^T P^T.
//  * lse_merge_frag / lse_merge: log-sum-exp merge of candidate splits.
#include "gfx950_mem.h"
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// 16 bytes -> EPL floats
template <typename T>
struct Vec;
template <>
struct Vec<float> {
    static constexpr int EPL = 4;
    __device__ static void widen(const uint4& u, float* f) {
        f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
    }
};
template <>
struct Vec<uint16_t> {
    static constexpr int EPL = 8;
    __device__ static void widen(const uint4& u, float* f) {
        f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
        f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
    }
};

// online-softmax merge of (m, l, o) states in log2 units
// Row of logical history position j of batch b in the K/V tensors: j itself (rows of the
// batch's own slice), or its physical row in the page pools when a block table is given;
// -1 when the table names a page outside the pools (the candidate is then skipped).
__device__ __forceinline__ int64_t kv_row(const AttnArgs& a, int b, int j) {
    if (!a.block_table) return j;
    const int64_t page = a.block_table[b * a.bt_stride + (j >> a.page_shift)];
    if (page < 0 || page >= (a.pool_rows >> a.page_shift)) return -1;
    return (page << a.page_shift) | (int64_t)(j & ((1 << a.page_shift) - 1));
}

// Pool rows of a candidate list: out[e] = the pool row of candidate e (kv_row), or -1 when
// the candidate is -1, out of range, not visible or on a page outside the pools.  One pass
// per call, so the multi-head kernel's workgroups (one per key/value head) read pool rows
// directly instead of each repeating the table lookups.
__global__ void __launch_bounds__(256) page_rows(AttnArgs a, int32_t* out) {
    const sa_problem& p = a.p;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)p.B * p.n_q * p.k) return;
    const long r = e / p.k;
    const int b = (int)(r / p.n_q), i = (int)(r % p.n_q);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const int j = a.idx[e];
    out[e] = (unsigned)j < (unsigned)L ? (int32_t)kv_row(a, b, j) : -1;
}

__device__ __forceinline__ void merge_state(float& m, float& l, float* o, int n, float m2, float l2, const float* o2) {
    const float mn = fmaxf(m, m2);
    const float a1 = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float a2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mn);
    l = l * a1 + l2 * a2;
    for (int e = 0; e < n; ++e) o[e] = o[e] * a1 + o2[e] * a2;
    m = mn;
}

// ------------------------------------------------------------------ attn_rows
template <typename T, int LPR, int G>
__global__ void __launch_bounds__(256) attn_rows(AttnArgs a) {
    constexpr int EPL = Vec<T>::EPL;
    constexpr int RPI = 64 / LPR;   // rows per load instruction
    constexpr int UNROLL = 8;       // load instructions in flight per operand
    constexpr int ROWS_IT = RPI * UNROLL;
    const sa_problem& p = a.p;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, rg = lane / LPR;

    // work item -> (b, i, hk), heads pinned to XCDs when Hkv % 8 == 0
    const long items = (long)p.B * p.n_q * p.Hkv;
    const long blk = blockIdx.x;
    int b, i, hk;
    {
        const int nib = (p.n_q + 3) / 4;
        const int wv = threadIdx.x >> 6;
        if (p.Hkv % 8 == 0) {
            const int xcd = (int)(blk % 8);
            const long local = blk / 8;
            const int hpx = p.Hkv / 8;
            hk = xcd + 8 * (int)(local % hpx);
            const long rest = local / hpx;
            b = (int)(rest / nib);
            i = (int)(rest % nib) * 4 + wv;
        } else {
            hk = (int)(blk % p.Hkv);
            const long rest = blk / p.Hkv;
            b = (int)(rest / nib);
            i = (int)(rest % nib) * 4 + wv;
        }
        if (b >= p.B || i >= p.n_q) return;
        (void)items;
    }
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const float sl2 = a.scale * kLog2e;

    const T* Qp = static_cast<const T*>(a.Q.data);
    const T* Kp = static_cast<const T*>(a.K.data);
    const T* Vp = static_cast<const T*>(a.V.data);
    float q[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int h = hk * G + g;
        uint4 u = *reinterpret_cast<const uint4*>(Qp + b * a.Q.s0 + h * a.Q.s1 + (int64_t)i * a.Q.s2 + sub * EPL);
        Vec<T>::widen(u, q[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) q[g][e] *= sl2;
    }
    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY; l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
    }
    const int32_t* ix = a.idx + ((int64_t)b * p.n_q + i) * p.k;
    const int64_t kbase = b * a.K.s0 + hk * a.K.s1 + sub * EPL;
    const int64_t vbase = b * a.V.s0 + hk * a.V.s1 + sub * EPL;

    if (L > 0) {
        for (int r0 = 0; r0 < p.k; r0 += ROWS_IT) {
            int jv[UNROLL];
            bool ok[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int r = r0 + u * RPI + rg;
                const int j = r < p.k ? ix[r] : -1;
                ok[u] = j >= 0 && j < L;
                jv[u] = ok[u] ? j : 0;
            }
            uint4 kr[UNROLL], vr[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                kr[u] = ok[u] ? *reinterpret_cast<const uint4*>(Kp + kbase + (int64_t)jv[u] * a.K.s2) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                vr[u] = ok[u] ? *reinterpret_cast<const uint4*>(Vp + vbase + (int64_t)jv[u] * a.V.s2) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float s[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    float kf[EPL];
                    Vec<T>::widen(kr[u], kf);
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = fmaf(q[g][e], kf[e], d);
#pragma unroll
                    for (int o2 = 1; o2 < LPR; o2 <<= 1) d += __shfl_xor(d, o2);
                    s[u] = ok[u] ? d : -INFINITY;
                }
                float mt = m[g];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) mt = fmaxf(mt, s[u]);
                // mt == -inf only if nothing was valid so far: then l, o are 0 and stay 0
                const float alpha = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - mt);
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const float pu = ok[u] ? exp2f(s[u] - mt) : 0.f;
                    l[g] += pu;
                    float vf[EPL];
                    Vec<T>::widen(vr[u], vf);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pu, vf[e], o[g][e]);
                }
                m[g] = mt;
            }
        }
    }
    // merge the RPI lane groups
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
            float m2 = __shfl_xor(m[g], off), l2 = __shfl_xor(l[g], off), o2[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) o2[e] = __shfl_xor(o[g][e], off);
            merge_state(m[g], l[g], o[g], EPL, m2, l2, o2);
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int h = hk * G + g;
            const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
            T* Op = static_cast<T*>(a.O.data) + b * a.O.s0 + h * a.O.s1 + (int64_t)i * a.O.s2 + sub * EPL;
            if constexpr (sizeof(T) == 4) {
                uint4 w;
                w.x = __float_as_uint(o[g][0] * inv); w.y = __float_as_uint(o[g][1] * inv);
                w.z = __float_as_uint(o[g][2] * inv); w.w = __float_as_uint(o[g][3] * inv);
                *reinterpret_cast<uint4*>(Op) = w;
            } else {
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pk[e] = (uint32_t)f32_to_bf16_rne(o[g][2 * e] * inv) | ((uint32_t)f32_to_bf16_rne(o[g][2 * e + 1] * inv) << 16);
                *reinterpret_cast<uint4*>(Op) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            }
            if (a.lse && sub == 0)
                a.lse[b * a.lse_bs + (int64_t)h * p.n_q + i] = l[g] > 0.f ? (m[g] + log2f(l[g])) * kLn2 : -INFINITY;
        }
    }
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// --------------------------------------------------------------- attn_tile
// bf16 MHA (d = 128) over selections that, for a block of query rows, cover most key tiles
// (many query rows, k a large fraction of the history).  One workgroup = 128 query rows of
// one head: the rows' selections become a bitmap (tile_bits), every 64-key tile that any of
// the rows selected is read once into LDS, S^T = K Q^T and O^T += V^T P^T run on MFMA
// (16x16x32 bf16), and unselected keys get probability 0, so each row's result is the exact
// softmax over its own selected set.  Tiles no row selected are skipped, and the V rows of
// keys that no row of the block selected enter LDS as zeros, so the value product never
// touches an unselected row, which may hold anything (padding, stale pool rows, NaN); an
// unselected K row only produces a logit that is masked.  Wave w owns query rows
// 16 w .. 16 w + 15.  With a block table the tile's keys are read from their pool rows
// (kv_row), and a candidate on a page outside the pools never enters the bitmap.
namespace tile {
constexpr int QR = 128;        // query rows per workgroup (16 per wave)
constexpr int NWV = QR / 16;   // waves per workgroup of the attention kernel
constexpr int KT = 64;         // keys per tile
constexpr int MAXN = 4096;     // longest history (bitmap words per row = MAXN / 32)
constexpr int D = 128;
static_assert(MAXN / KT <= 64, "a row block's tile list fits one register per wave");
// LDS rows are not padded (256 B per K or V row; K and V double-buffered, 64 KB per workgroup,
// so two workgroups of eight waves share a CU); the 16-byte chunks of a row are XOR-swizzled
// instead.  K: chunk c of row r at
// slot c ^ (r & 15), so the 16-row operand reads touch distinct banks.  V: slot c ^ 2 (r & 7),
// so each transposing read (16 rows x two adjacent chunks, half a wave per pass) touches
// every bank once per pass.
__device__ __forceinline__ int kslot(int row, int chunk) { return chunk ^ (row & 15); }
__device__ __forceinline__ int vslot(int row, int chunk) { return chunk ^ (2 * (row & 7)); }
// The selections pre-pass works on blocks of SUB rows (more workgroups than the attention's
// QR-row blocks); per SUB-row block: [0, 1] the 64-bit mask of tiles that any of its rows
// selected, then for tile t at [2 + 2 t, 3 + 2 t] the union over its rows of that tile's
// selection bits
constexpr int SUB = 64;
constexpr int LIST = 2 + 2 * KT;
static_assert(QR % SUB == 0, "an attention row block is whole selection blocks");
constexpr float kLazy = 0x1p64f;  // exp2(64): largest probability against a row's reference
}  // namespace tile

// The selections of a batch's block of SUB query rows, shared by every head: a bitmap per
// row (bit j of word j / 32 = position j selected), the mask of 64-key tiles any of the
// rows selected and, per tile, the union of the rows' selection bits.  One workgroup per
// (batch, row block); written to the workspace.
__global__ void __launch_bounds__(1024) tile_bits(AttnArgs a, uint32_t* gbits, int32_t* glist) {
    using namespace tile;
    constexpr int NWORD = MAXN / 32;
    constexpr int NT = 1024;
    constexpr int QR = SUB;  // rows of this pre-pass block
    __shared__ __attribute__((aligned(16))) uint32_t bits[QR][NWORD];
    __shared__ int s_L[QR], s_maxL;
    __shared__ uint32_t s_uni[NT / 64][KT][2];
    const sa_problem& p = a.p;
    const int tid = threadIdx.x, lane = tid & 63;
    const int nqb = (p.n_q + QR - 1) / QR;
    const int b = (int)(blockIdx.x / nqb), qb = (int)(blockIdx.x % nqb);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    if (tid < QR) {
        const int i = qb * QR + tid;
        s_L[tid] = i < p.n_q ? visible_len(R, b, i) : 0;
    }
    for (int w = tid; w < QR * NWORD; w += NT) (&bits[0][0])[w] = 0u;
    if (tid == 0) s_maxL = 0;
    __syncthreads();
    if (tid < QR) atomicMax(&s_maxL, s_L[tid]);
    {   // TPR threads per row, eight 16-byte index loads in flight per thread
        constexpr int TPR = NT / QR;
        const int r = tid / TPR, q = tid % TPR;
        const int i = qb * QR + r, L = s_L[r];
        if (i < p.n_q && L > 0) {
            const int32_t* ix = a.idx + ((int64_t)b * p.n_q + i) * p.k;
            for (int e0 = 4 * q; e0 < p.k; e0 += 4 * TPR * 8) {
                int4 jj[8];
#pragma unroll
                for (int n = 0; n < 8; ++n)
                    jj[n] = e0 + 4 * TPR * n < p.k ? *reinterpret_cast<const int4*>(ix + e0 + 4 * TPR * n) : make_int4(-1, -1, -1, -1);
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const int jv[4] = {jj[n].x, jj[n].y, jj[n].z, jj[n].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if ((unsigned)jv[u] < (unsigned)L && (!a.block_table || kv_row(a, b, jv[u]) >= 0))
                            atomicOr(&bits[r][jv[u] >> 5], 1u << (jv[u] & 31));
                }
            }
        }
    }
    __syncthreads();
    const int ntile = (s_maxL + KT - 1) / KT;
    {   // union over QR / 16 rows per thread, then over the sixteen row groups
        constexpr int RG = QR / (NT / 64);
        const int t = tid & 63, rq = tid >> 6;
        uint32_t u0 = 0, u1 = 0;
        if (t < ntile)
#pragma unroll
            for (int r = RG * rq; r < RG * rq + RG; ++r) {
                u0 |= bits[r][2 * t];
                u1 |= bits[r][2 * t + 1];
            }
        s_uni[rq][t][0] = u0;
        s_uni[rq][t][1] = u1;
    }
    __syncthreads();
    int32_t* list = glist + (size_t)(b * nqb + qb) * LIST;
    if (tid < 64) {
        uint32_t u0 = 0, u1 = 0;
#pragma unroll
        for (int rq = 0; rq < NT / 64; ++rq) {
            u0 |= s_uni[rq][lane][0];
            u1 |= s_uni[rq][lane][1];
        }
        const uint64_t m = __ballot((u0 | u1) != 0);
        list[2 + 2 * lane] = (int32_t)u0;
        list[3 + 2 * lane] = (int32_t)u1;
        if (lane == 0) {
            list[0] = (int32_t)(uint32_t)m;
            list[1] = (int32_t)(uint32_t)(m >> 32);
        }
    }
    // the rows' bitmaps, as 16-byte pieces
    for (int w = tid; w < QR * NWORD / 4; w += NT) {
        const int r = w / (NWORD / 4), c = w % (NWORD / 4);
        const int i = qb * QR + r;
        if (i < p.n_q)
            reinterpret_cast<uint4*>(gbits + ((size_t)b * p.n_q + i) * NWORD)[c] = reinterpret_cast<const uint4*>(bits[r])[c];
    }
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short v4s __attribute__((ext_vector_type(4)));

// maximum over the lanes l, l^16, l^32, l^48 (lane swaps between rows, no LDS round trip)
__device__ __forceinline__ float colmax4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ v4s lds_tr_read(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
}

template <int N>
struct ICst {
    static constexpr int value = N;
};

// Zeros that stand in for a row no lane may read (an unselected or unmapped pool row)
constexpr int kZeroRowBytes = 4096;
__device__ __align__(16) const uint8_t kZeroRow[kZeroRowBytes] = {};

// The tile kernel.  S^T = K Q^T leaves one query row in each lane (keys 16 j + 4 g + e of the
// tile in its accumulators), so the row's mask bits come from its own bitmap word, the
// softmax needs no lane exchange unless a row's reference maximum moves, and the
// probabilities are already the B operand of O^T += V^T P^T (no LDS round trip).  K and V
// tiles reach LDS through loads that write LDS directly (K of tile u + 1 while tile u's
// values are used, V of tile u + 1 while its scores run); V^T operands come from transposing
// LDS reads of the row-major tile.  A row's reference maximum is raised only when one of its
// selected logits exceeds it by more than 64 (exp2 units): below that margin every
// probability and sum stays far inside fp32 range, and any reference gives the same
// softmax.  A row's sum is kept per lane in fp32 (from the unrounded probabilities) and
// added over the row's four lanes at the end.
// Tile sources: contiguous K/V and pages of at least 64 rows give each tile one contiguous
// run of rows, read through a buffer resource made per tile (rows past the history read
// zeros); ROWS (pages shorter than a tile) looks up each row's pool row and reads it by its
// own 64-bit address, unselected rows from the zero row.
template <bool ROWS>
__global__ void __launch_bounds__(64 * tile::NWV) __attribute__((amdgpu_waves_per_eu(3)))
attn_tile(AttnArgs a, const uint32_t* gbits, const int32_t* glist) {
    using namespace tile;
    constexpr int NWORD = MAXN / 32;
    constexpr int TB = KT * D * 2;  // bytes of one K or V tile
    __shared__ __attribute__((aligned(16))) uint8_t Ks[2 * TB];
    __shared__ __attribute__((aligned(16))) uint8_t Vs[2 * TB];
    const sa_problem& p = a.p;
    const int tid = threadIdx.x, lane = tid & 63, l15 = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nqb = (p.n_q + QR - 1) / QR;
    int b, h, qb;
    {
        const long blk = blockIdx.x;
        long rest;
        // the longest (latest) row blocks first; with Hkv % 8 == 0 each XCD keeps to heads
        // h = XCD (mod 8), so those heads' K/V stay in its L2
        if (p.Hkv % 8 == 0) {
            const long local = blk / 8;
            const int hb = (p.Hkv / 8) * p.B;  // (head, batch) pairs per XCD
            const int rr = (int)(local % hb);
            h = (int)(blk % 8) + 8 * (rr / p.B);
            b = rr % p.B;
            qb = nqb - 1 - (int)(local / hb);
        } else {
            h = (int)(blk % p.Hkv);
            rest = blk / p.Hkv;
            b = (int)(rest / nqb);
            qb = nqb - 1 - (int)(rest % nqb);
        }
    }
    // the block's active tiles (mask) and, in lane t, tile t's union of selection bits: ORed
    // over the block's selection blocks
    uint64_t tmask = 0;
    uint32_t lu0 = 0u, lu1 = 0u;
    {
        const int nsb = (p.n_q + SUB - 1) / SUB;
#pragma unroll
        for (int k = 0; k < QR / SUB; ++k) {
            const int sb = qb * (QR / SUB) + k;
            if (sb < nsb) {
                const int32_t* list = glist + (size_t)(b * nsb + sb) * LIST;
                tmask |= (uint64_t)(uint32_t)list[0] | ((uint64_t)(uint32_t)list[1] << 32);
                lu0 |= (uint32_t)list[2 + 2 * lane];
                lu1 |= (uint32_t)list[3 + 2 * lane];
            }
        }
        tmask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tmask)) |
                ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tmask >> 32)) << 32);
    }
    const int nt = __popcll(tmask);
    const int iq = qb * QR + 16 * wv + l15;  // this lane's query row
    const char* Kb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.K.data) + (a.block_table ? 0 : b * a.K.s0) + h * a.K.s1);
    const char* Vb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.V.data) + (a.block_table ? 0 : b * a.V.s0) + h * a.V.s1);
    const int64_t krow = a.K.s2 * 2, vrow = a.V.s2 * 2;  // bytes per row
    // the block's bitmap rows; rows past n_q read zeros
    const int nrows = min(QR, p.n_q - qb * QR);
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(gbits + ((size_t)b * p.n_q + (size_t)qb * QR) * NWORD), (short)0, nrows * (NWORD * 4), 0x00020000);
    const uint32_t boff = (uint32_t)(16 * wv + l15) * (NWORD * 4);

    // Q^T fragments (B operand of S^T): query row iq, d = 32 s + 8 g .. + 7
    bf16x8 qa[D / 32];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.Q.data) + b * a.Q.s0 + h * a.Q.s1 + (int64_t)min(iq, p.n_q - 1) * a.Q.s2;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            qa[s] = iq < p.n_q ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g))
                               : bf16x8{};
    }
    // tile loads: wave wv fills the 1 KB LDS blocks LPW wv + i, i.e. tile rows r_i = 4 (LPW wv + i)
    // + lane / 16, lane l writing slot l % 16 of its row (the chunk whose swizzled slot that is)
    constexpr int LPW = 16 / NWV;  // 1 KB blocks per wave and tile
    uint32_t koff[LPW], voff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int r = 4 * (LPW * wv + i) + (lane >> 4);
        koff[i] = 16u * (uint32_t)kslot(r, lane & 15);
        voff[i] = 16u * (uint32_t)vslot(r, lane & 15);
        if constexpr (!ROWS) {
            koff[i] += (uint32_t)(r * krow);
            voff[i] += (uint32_t)(r * vrow);
        }
    }
    const uint32_t kl = lds_addr(Ks) + 1024u * LPW * (uint32_t)wv, vl = lds_addr(Vs) + 1024u * LPW * (uint32_t)wv;
    // where a tile's rows come from: a per-tile buffer resource, or (ROWS) each row's pool row
    struct Src {
        v4i krs, vrs;
        int64_t prow[LPW];
    };
    auto tile_src = [&](int k0, uint64_t uni) {
        Src t;
        if constexpr (ROWS) {
            const uint64_t un = uni >> (4 * LPW * wv);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int r = 4 * i + (lane >> 4);
                t.prow[i] = ((un >> r) & 1u) ? kv_row(a, b, k0 + 4 * LPW * wv + r) : -1;
            }
        } else {
            int64_t r0;
            int n;
            if (a.block_table) {  // the tile lies inside one page
                r0 = kv_row(a, b, k0);
                n = r0 >= 0 ? KT : 0;
            } else {
                r0 = k0;
                n = min(KT, p.n_kv - k0);
            }
            t.krs = buffer_rsrc(Kb + max(r0, (int64_t)0) * krow, (uint32_t)(n * krow));
            t.vrs = buffer_rsrc(Vb + max(r0, (int64_t)0) * vrow, (uint32_t)(n * vrow));
        }
        return t;
    };
    // K and V of a tile into LDS buffer bf
    auto issue = [&](const Src& t, uint64_t uni, int bf) {
        const uint32_t kb = kl + (uint32_t)(TB * bf), vb = vl + (uint32_t)(TB * bf);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            if constexpr (ROWS)
                lds_dma16_g(kb + 1024u * (uint32_t)i, t.prow[i] >= 0 ? Kb + t.prow[i] * krow + koff[i] : reinterpret_cast<const char*>(kZeroRow));
            else
                lds_dma16(t.krs, kb + 1024u * (uint32_t)i, koff[i], 0u);
        }
        const uint64_t un = uni >> (4 * LPW * wv);
        constexpr uint32_t ALL = (1u << (4 * LPW)) - 1u;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            if constexpr (ROWS) {
                lds_dma16_g(vb + 1024u * (uint32_t)i, t.prow[i] >= 0 ? Vb + t.prow[i] * vrow + voff[i] : reinterpret_cast<const char*>(kZeroRow));
            } else if (((uint32_t)un & ALL) == ALL) {  // every row of this wave's part selected
                lds_dma16(t.vrs, vb + 1024u * (uint32_t)i, voff[i], 0u);
            } else {
                // keys no row of the block selected read past the resource: zeros
                const bool sel = ((uint32_t)(un >> (4 * i)) >> (lane >> 4)) & 1u;
                lds_dma16(t.vrs, vb + 1024u * (uint32_t)i, sel ? voff[i] : 0x80000000u, 0u);
            }
        }
    };
    auto load_bits = [&](int k0) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(brs, boff + 4u * (uint32_t)(k0 >> 5), 0, 0);
        return make_uint2(v[0], v[1]);
    };
    // LDS read offsets.  K (A operand of S^T: key 16 j + l15, chunk 4 s + g): kad[s] + 4096 j.
    // V^T (A operand of O^T by transposing reads): this lane supplies row 32 s + 16 hf + rr,
    // rr = 4 g + l15 / 4, and 8 bytes at column 16 t + 4 (l15 % 4): vad[t] + 8192 s + 4096 hf
    int kad[D / 32], vad[D / 16];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) kad[s] = 256 * l15 + 16 * kslot(l15, 4 * s + g);
    {
        const int rr = 4 * g + (l15 >> 2);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) vad[t] = 256 * rr + 16 * vslot(rr, 2 * t + ((l15 >> 1) & 1)) + 8 * (l15 & 1);
    }

    const float sl2 = a.scale * kLog2e;
    float ref = -INFINITY;  // reference maximum of row iq (scaled log2 units)
    bool all_ref = false;   // every valid row of the wave has a finite reference
    float lrow = 0.f;       // this lane's part of the row's sum (keys 16 j + 4 g + e)
    f32x4 o[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // active tiles in ascending order: tile u is the lowest set bit of rem after u steps
    uint64_t rem = tmask;
    auto tile_union = [&](int t) {
        return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lu0, t) | ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lu1, t) << 32);
    };
    uint2 wcur = make_uint2(0u, 0u);
    if (nt > 0) {
        const int t0 = __builtin_ctzll(rem);
        rem &= rem - 1;
        const int k0 = t0 * KT;
        const uint64_t un = tile_union(t0);
        issue(tile_src(k0, un), un, 0);
        wcur = load_bits(k0);
        wait_vmcnt<0>();
        tile_barrier();
    }
    // one tile: the next tile's K, V (other buffer) and bitmap words are issued first and have
    // the whole tile's work to land; one barrier per tile
    auto step = [&](auto BFC) {
        constexpr int BF = decltype(BFC)::value;
        const bool more = rem != 0;
        const int t1 = more ? __builtin_ctzll(rem) : 0;
        rem &= rem - 1;
        uint2 wnext = make_uint2(0u, 0u);
        if (more) {
            const int k1 = t1 * KT;
            const uint64_t un1 = tile_union(t1);
            issue(tile_src(k1, un1), un1, 1 - BF);
            wnext = load_bits(k1);
        }
        // does any row of this wave select a key of the tile?
        const bool act = __ballot((wcur.x | wcur.y) != 0u) != 0;
        // S^T = K Q^T: acc[j][e] = S[row iq][key 16 j + 4 g + e]
        f32x4 acc[4];
        if (act) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 kb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ks + TB * BF + kad[s] + 4096 * j));
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qa[s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[j], 0, 0, 0);
                }
            // mask of row iq for keys 16 j + 4 g + e: bit 16 (j % 2) + e of word j / 2 after a shift
            // by 4 g; all ones where selected (one bit-field extract, kept opaque so that the
            // masking stays a single AND per element)
            const uint32_t w0 = wcur.x >> (4 * g), w1 = wcur.y >> (4 * g);
            auto msk = [&](int j, int e) -> uint32_t {
                uint32_t m;
                asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(j < 2 ? w0 : w1), "i"(16 * (j & 1) + e));
                return m;
            };
            float pr[4][4];
            auto probs = [&](float nref) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pr[j][e] = __uint_as_float(__float_as_uint(__builtin_amdgcn_exp2f(fmaf(acc[j][e], sl2, nref))) & msk(j, e));
            };
            bool slow = !all_ref;
            if (!slow) {
                probs(-ref);
                // largest probability of the lane, compared as bit patterns (all are >= +0; inf and
                // NaN order above every finite value and so take the slow path too)
                uint32_t pm = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pm = max(max(pm, max(__float_as_uint(pr[j][0]), __float_as_uint(pr[j][1]))),
                             max(__float_as_uint(pr[j][2]), __float_as_uint(pr[j][3])));
                slow = __ballot(pm > __float_as_uint(kLazy)) != 0;
            }
            if (slow) {
                // the row's maximum over its selected keys (all four lanes of the row)
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t m = msk(j, e);
                        mx = fmaxf(mx, __uint_as_float((__float_as_uint(acc[j][e] * sl2) & m) | (0xff800000u & ~m)));
                    }
                const float mn = fmaxf(ref, colmax4(mx));
                const float alpha = ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ref - mn);
#pragma unroll
                for (int t = 0; t < D / 16; ++t) o[t] *= alpha;
                lrow *= alpha;
                ref = mn;
                all_ref = __ballot(iq < p.n_q && ref == -INFINITY) == 0;
                probs(ref == -INFINITY ? 0.f : -ref);
            }
            float ps = (pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3]);
#pragma unroll
            for (int j = 1; j < 4; ++j) ps += (pr[j][0] + pr[j][1]) + (pr[j][2] + pr[j][3]);
            lrow += ps;
            // P^T fragments (B operand): k-step s holds keys 32 s + 4 g + 0..3, then 32 s + 16 + 4 g + 0..3
            bf16x8 pb[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pb[s][e] = (__bf16)pr[2 * s][e];
                    pb[s][4 + e] = (__bf16)pr[2 * s + 1][e];
                }
            // O^T[d 16 t + 4 g + e][row iq] += V^T P^T; the first of a pair of transposing reads
            // brings keys 32 s + 4 g + 0..3 of column 16 t + l15, the second 32 s + 16 + 4 g + 0..3
            auto vread = [&](int s, int t) {
                const uint8_t* vp = Vs + TB * BF + vad[t] + 8192 * s;
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lds_tr_read(vp), lds_tr_read(vp + 4096), 0, 1, 2, 3, 4, 5, 6, 7));
            };
            // (raised issue priority while the value products run, so that this wave's MFMAs and
            // transposing reads go ahead of the other waves' softmax arithmetic)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int t = 0; t < D / 16; ++t) o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vread(s, t), pb[s], o[t], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        }
        wait_lgkmcnt0();
        wait_vmcnt<0>();  // this wave's part of the next tile and its bitmap words have landed
        tile_barrier();   // every wave is done with buffer BF; the next tile is complete
        wcur = wnext;
    };
    for (int u = 0; u < nt; u += 2) {
        step(ICst<0>{});
        if (u + 1 < nt) step(ICst<1>{});
    }
    // O[row iq][d 16 t + 4 g + e] = O^T / l; LSE per row
    float l;
    {
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(lrow), __float_as_uint(lrow), false, false);
        const float y = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
        l = __uint_as_float(z[0]) + __uint_as_float(z[1]);
    }
    if (iq < p.n_q) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* op = static_cast<uint16_t*>(a.O.data) + b * a.O.s0 + h * a.O.s1 + (int64_t)iq * a.O.s2;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) op[16 * t + 4 * g + e] = f32_to_bf16_rne(o[t][e] * inv);
        if (a.lse && g == 0) a.lse[b * a.lse_bs + (int64_t)h * p.n_q + iq] = l > 0.f ? (ref + log2f(l)) * kLn2 : -INFINITY;
    }
}

// --------------------------------------------------------------- attn_rows_buf
// bf16, one query head per key/value head, head width D.  Loads stay coalesced and the
// arithmetic stays in the VALU (the contraction is a GEMV per candidate set):
//  * K and V rows are fetched with raw buffer loads on a per-(batch, head) resource, so a
//    row address is one 32-bit multiply; an invalid entry gets an offset past the end of
//    the resource and the hardware returns zeros (no branches, no zero-fill moves);
//  * each lane covers 32 bytes (16 elements) of a row in two 16-byte pieces, one in each
//    half-row, so every load instruction reads whole contiguous half-rows; LPR = D/16
//    lanes per row; q.k uses v_dot2_f32_bf16 and an LPR-lane sum of DPP moves (quad swaps,
//    half-row and row mirrors); p.V runs as v_dot2_f32_bf16 on pairs of rows interleaved by
//    v_perm_b32 (probabilities rounded to bf16, fp32 accumulation);
//  * row group rg takes UNROLL consecutive candidate entries, fetched by one 16-byte load;
//  * exponentials use v_exp_f32 directly on arguments <= 0.
// Requires k % 4 == 0 and every (batch, head) slice of K and V below 2^31 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int LPR>
__device__ __forceinline__ float group_sum2(float x) {
    if constexpr (LPR >= 2) x += dpp_mov<0xB1>(x);
    if constexpr (LPR >= 4) x += dpp_mov<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);
    if constexpr (LPR >= 16) x += dpp_mov<0x140>(x);
    return x;
}

// PAGED: the candidate list holds pool rows already (page_rows below), -1 for a skipped slot.
template <int D, bool PAGED>
__global__ void __launch_bounds__(256) attn_rows_buf(AttnArgs a) {
    constexpr int LPR = D / 16;      // lanes per row, 32 bytes each
    constexpr int RPG = 64 / LPR;    // row groups per wave
    constexpr int UNROLL = 4;        // rows per row group per iteration
    constexpr int ROWS_IT = RPG * UNROLL;
    const sa_problem& p = a.p;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, rg = lane / LPR;

    const long blk = blockIdx.x;
    int b, i, hk;
    {
        const int nib = (p.n_q + 3) / 4;
        const int wv = threadIdx.x >> 6;
        if (p.Hkv % 8 == 0) {  // one head at a time per XCD: its K/V rows stay in that L2
            const int xcd = (int)(blk % 8);
            const long local = blk / 8;
            hk = xcd + 8 * (int)(local / ((long)p.B * nib));
            const long rest = local % ((long)p.B * nib);
            b = (int)(rest / nib);
            i = (int)(rest % nib) * 4 + wv;
        } else {
            hk = (int)(blk % p.Hkv);
            const long rest = blk / p.Hkv;
            b = (int)(rest / nib);
            i = (int)(rest % nib) * 4 + wv;
        }
        if (b >= p.B || i >= p.n_q) return;
    }
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const float sl2 = a.scale * kLog2e;
    const int h = hk;

    // lane `sub` owns elements [8 sub, 8 sub + 8) and [D/2 + 8 sub, D/2 + 8 sub + 8): each of its
    // two 16-byte loads is part of one contiguous half-row read by the LPR lanes together
    constexpr int HALF = D / 2;
    const uint16_t* Qp = static_cast<const uint16_t*>(a.Q.data) + b * a.Q.s0 + h * a.Q.s1 + (int64_t)i * a.Q.s2 + 8 * sub;
    const uint4 qa = *reinterpret_cast<const uint4*>(Qp), qc = *reinterpret_cast<const uint4*>(Qp + HALF);
    const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qc.x, qc.y, qc.z, qc.w};
    const uint32_t kstride = (uint32_t)(a.K.s2 * 2), vstride = (uint32_t)(a.V.s2 * 2);
    const int64_t kb0 = PAGED ? 0 : b * a.K.s0, vb0 = PAGED ? 0 : b * a.V.s0;
    const uint32_t nrows = (uint32_t)(PAGED ? a.pool_rows : p.n_kv);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(static_cast<const uint16_t*>(a.K.data) + kb0 + hk * a.K.s1, nrows * kstride);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const uint16_t*>(a.V.data) + vb0 + hk * a.V.s1, nrows * vstride);
    const int32_t* ix = a.idx + ((int64_t)b * p.n_q + i) * p.k;
    const uint32_t col = 16u * sub;

    float m = -INFINITY, l = 0.f, o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;

    for (int r0 = 0; L > 0 && r0 < p.k; r0 += ROWS_IT) {
        const int rb = r0 + UNROLL * rg;
        int4 jj = rb < p.k ? *reinterpret_cast<const int4*>(ix + rb) : make_int4(-1, -1, -1, -1);
        const int jv[UNROLL] = {jj.x, jj.y, jj.z, jj.w};
        uint32_t koff[UNROLL], voff[UNROLL];
        bool ok[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            ok[u] = PAGED ? jv[u] >= 0 : (unsigned)jv[u] < (unsigned)L;
            koff[u] = ok[u] ? __umul24((uint32_t)jv[u], kstride) + col : 0x80000000u;
            voff[u] = ok[u] ? __umul24((uint32_t)jv[u], vstride) + col : 0x80000000u;
        }
        uint32_t kw[UNROLL][8], vw[UNROLL][8];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            auto k0 = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[u], 0, 0);
            auto k1 = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[u] + HALF * 2, 0, 0);
#pragma unroll
            for (int w = 0; w < 4; ++w) { kw[u][w] = k0[w]; kw[u][4 + w] = k1[w]; }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            auto v0 = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[u], 0, 0);
            auto v1 = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[u] + HALF * 2, 0, 0);
#pragma unroll
            for (int w = 0; w < 4; ++w) { vw[u][w] = v0[w]; vw[u][4 + w] = v1[w]; }
        }
        float x[UNROLL];
        float mt = m;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float d = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w)
                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[w]), __builtin_bit_cast(bf16x2, kw[u][w]), d, false);
            d = group_sum2<LPR>(d);
            x[u] = ok[u] ? d * sl2 : -INFINITY;
            mt = fmaxf(mt, x[u]);
        }
        // mt == -inf only if nothing was valid so far: then l, o are 0 and stay 0
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mt);
        const float mref = (mt == -INFINITY) ? 0.f : mt;  // keeps exp2(x - mref) = 0, never NaN
        float pr[UNROLL];
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            pr[u] = __builtin_amdgcn_exp2f(x[u] - mref);  // exp2(-inf) = 0 for invalid rows
            ps += pr[u];
        }
        l = l * alpha + ps;
        m = mt;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < UNROLL; u += 2) {
            const bf16x2 pw = {(__bf16)pr[u], (__bf16)pr[u + 1]};
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint32_t lo = __builtin_amdgcn_perm(vw[u + 1][w], vw[u][w], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(vw[u + 1][w], vw[u][w], 0x07060302u);
                o[2 * w] = __builtin_amdgcn_fdot2_f32_bf16(pw, __builtin_bit_cast(bf16x2, lo), o[2 * w], false);
                o[2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(pw, __builtin_bit_cast(bf16x2, hi), o[2 * w + 1], false);
            }
        }
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off), o2[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) o2[e] = __shfl_xor(o[e], off);
        merge_state(m, l, o, 16, m2, l2, o2);
    }
    if (rg == 0) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* Op = static_cast<uint16_t*>(a.O.data) + b * a.O.s0 + h * a.O.s1 + (int64_t)i * a.O.s2 + 8 * sub;
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pk[e] = (uint32_t)f32_to_bf16_rne(o[2 * e] * inv) | ((uint32_t)f32_to_bf16_rne(o[2 * e + 1] * inv) << 16);
        *reinterpret_cast<uint4*>(Op) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        *reinterpret_cast<uint4*>(Op + HALF) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        if (a.lse && sub == 0)
            a.lse[b * a.lse_bs + (int64_t)h * p.n_q + i] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
}

// Split partials: (m, l) pairs in fp32 for every (row, head, split), then, from the next
// 256-byte boundary, o / l in bf16 (d_v values per (row, head, split)).
__device__ __forceinline__ uint16_t* partial_o(float* part, int64_t slots) {
    return reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(part) + ((slots * 8 + 255) & ~(int64_t)255));
}
__device__ __forceinline__ const uint16_t* partial_o(const float* part, int64_t slots) {
    return partial_o(const_cast<float*>(part), slots);
}

// ------------------------------------------------------------------- attn_mla
constexpr int kTile = 32;

__device__ __forceinline__ int vt_slot(int pos) {  // position in tile -> lane-ordered slot
    const int mt = pos >> 4, g = (pos >> 2) & 3, r = pos & 3;
    return 8 * g + 4 * mt + r;
}

template <int DQK, int DV>
__global__ void __launch_bounds__(512) attn_mla(AttnArgs a) {
    constexpr int KS = DQK / 32;          // k-steps of S^T
    constexpr int KPAD = DQK + 8;         // LDS row pitch of the K tile (elements)
    constexpr int VTP = kTile + 8;        // LDS row pitch of the transposed V tile (elements)
    constexpr int MTV = DV / 16;          // 16-row tiles of O^T
    constexpr int CH = DQK / 8;           // 16-byte chunks per K row
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t VT[DV * VTP];
    __shared__ int s_j[kTile];

    const sa_problem& p = a.p;
    const int nw = blockDim.x >> 6;  // waves = heads per kv head / 16
    const int G = p.Hq / p.Hkv;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, gq = lane >> 4;
    const int S = a.splits;
    const long unit = blockIdx.x;  // (b, i, hk, split)
    const int split = (int)(unit % S);
    const long rowkv = unit / S;
    const int hk = (int)(rowkv % p.Hkv);
    const long row = rowkv / p.Hkv;
    const int b = (int)(row / p.n_q), i = (int)(row % p.n_q);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const int head = hk * G + 16 * wv + c;  // this lane's query head (column of S^T)
    const bool v_alias = a.V.data == a.K.data;

    // Q^T fragments: B operand of S^T, lane (gq, c): head c, d = 32 s + 8 gq
    bf16x8 bq[KS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.Q.data) + b * a.Q.s0 + head * a.Q.s1 + (int64_t)i * a.Q.s2;
#pragma unroll
        for (int s = 0; s < KS; ++s) bq[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * gq));
    }
    f32x4 oacc[MTV];
#pragma unroll
    for (int t = 0; t < MTV; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    const float sl2 = a.scale * kLog2e;

    const int per = (p.k + S - 1) / S;
    const int e_begin = split * per, e_end = min(p.k, e_begin + per);
    const int32_t* ix = a.idx + row * (int64_t)p.k;
    const uint16_t* Kg = static_cast<const uint16_t*>(a.K.data) + b * a.K.s0 + hk * a.K.s1;
    const uint16_t* Vg = static_cast<const uint16_t*>(a.V.data) + b * a.V.s0 + hk * a.V.s1;

    for (int t0 = e_begin; L > 0 && t0 < e_end; t0 += kTile) {
        if (threadIdx.x < kTile) {
            const int e = t0 + threadIdx.x;
            int j = e < e_end ? ix[e] : -1;
            s_j[threadIdx.x] = (j >= 0 && j < L) ? j : -1;
        }
        __syncthreads();
        // stage K rows (row-major) and V rows (transposed, lane-ordered slots).  A thread
        // takes one 16-byte chunk of two adjacent positions, which share a 32-bit word in
        // every transposed row.
        for (int q = threadIdx.x; q < (kTile / 2) * CH; q += blockDim.x) {
            const int pp = q % (kTile / 2), ch = q / (kTile / 2);
            const int p0 = 2 * pp;
            const int j0 = s_j[p0], j1 = s_j[p0 + 1];
            const uint4 u0 = j0 >= 0 ? *reinterpret_cast<const uint4*>(Kg + (int64_t)j0 * a.K.s2 + 8 * ch) : make_uint4(0, 0, 0, 0);
            const uint4 u1 = j1 >= 0 ? *reinterpret_cast<const uint4*>(Kg + (int64_t)j1 * a.K.s2 + 8 * ch) : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(&Ks[p0 * KPAD + 8 * ch]) = u0;
            *reinterpret_cast<uint4*>(&Ks[(p0 + 1) * KPAD + 8 * ch]) = u1;
            if (ch < DV / 8) {
                uint4 v0 = u0, v1 = u1;
                if (!v_alias) {
                    v0 = j0 >= 0 ? *reinterpret_cast<const uint4*>(Vg + (int64_t)j0 * a.V.s2 + 8 * ch) : make_uint4(0, 0, 0, 0);
                    v1 = j1 >= 0 ? *reinterpret_cast<const uint4*>(Vg + (int64_t)j1 * a.V.s2 + 8 * ch) : make_uint4(0, 0, 0, 0);
                }
                const int sl = vt_slot(p0);  // vt_slot(p0 + 1) == sl + 1 since p0 is even
                const uint32_t a4[4] = {v0.x, v0.y, v0.z, v0.w}, b4[4] = {v1.x, v1.y, v1.z, v1.w};
                uint32_t* vt32 = reinterpret_cast<uint32_t*>(VT);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vt32[((8 * ch + 2 * e) * VTP + sl) >> 1] = (a4[e] & 0xffffu) | (b4[e] << 16);
                    vt32[((8 * ch + 2 * e + 1) * VTP + sl) >> 1] = (a4[e] >> 16) | (b4[e] & 0xffff0000u);
                }
            }
        }
        __syncthreads();
        // S^T = K Q^T: two 16-position M-tiles
        f32x4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t* kr = &Ks[(16 * mt + c) * KPAD + 8 * gq];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + 32 * s));
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[s], sacc[mt], 0, 0, 0);
            }
        }
        // lane holds S^T[pos 16 mt + 4 gq + r][head c]
        float x[8];
        float mt_max = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pos = 16 * mt + 4 * gq + r;
                const float v = s_j[pos] >= 0 ? sacc[mt][r] * sl2 : -INFINITY;
                x[4 * mt + r] = v;
                mt_max = fmaxf(mt_max, v);
            }
        mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 16));
        mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 32));
        const float mn = fmaxf(m, mt_max);
        if (mn == -INFINITY) {
            __syncthreads();
            continue;
        }
        const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
        m = mn;
        float pv[8];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = x[e] == -INFINITY ? 0.f : exp2f(x[e] - mn);
            ps += pv[e];
        }
        lsum = lsum * alpha + ps;
        bf16x8 pb;
        {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)f32_to_bf16_rne(pv[2 * e]) | ((uint32_t)f32_to_bf16_rne(pv[2 * e + 1]) << 16);
            pb = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
        // O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < MTV; ++t) {
            oacc[t][0] *= alpha; oacc[t][1] *= alpha; oacc[t][2] *= alpha; oacc[t][3] *= alpha;
            bf16x8 va = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&VT[(16 * t + c) * VTP + 8 * gq]));
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[t], 0, 0, 0);
        }
        __syncthreads();
    }
    // total exp-sum per head: lanes with the same c hold disjoint positions
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    // lane holds O^T[d = 16 t + 4 gq + r][head c]
    if (S == 1) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        uint16_t* op = static_cast<uint16_t*>(a.O.data) + b * a.O.s0 + head * a.O.s1 + (int64_t)i * a.O.s2;
#pragma unroll
        for (int t = 0; t < MTV; ++t) {
            const uint32_t lo = (uint32_t)f32_to_bf16_rne(oacc[t][0] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[t][1] * inv) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_rne(oacc[t][2] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[t][3] * inv) << 16);
            *reinterpret_cast<uint2*>(op + 16 * t + 4 * gq) = make_uint2(lo, hi);
        }
        if (a.lse && gq == 0)
            a.lse[b * a.lse_bs + (int64_t)head * p.n_q + i] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
    } else {
        // partial: [row, Hq, S] x (m, l) fp32, then [row, Hq, S, DV] o / l in bf16
        float* part = static_cast<float*>(a.partial);
        const int64_t slot = (row * p.Hq + head) * (int64_t)S + split;
        float* ml = part + slot * 2;
        uint16_t* po = partial_o(part, (int64_t)p.B * p.n_q * p.Hq * S) + slot * DV;
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
        for (int t = 0; t < MTV; ++t) {
            const uint32_t lo = (uint32_t)f32_to_bf16_rne(oacc[t][0] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[t][1] * inv) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_rne(oacc[t][2] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[t][3] * inv) << 16);
            *reinterpret_cast<uint2*>(po + 16 * t + 4 * gq) = make_uint2(lo, hi);
        }
        if (gq == 0) {
            ml[0] = m;
            ml[1] = lsum;
        }
    }
}

// Merge the S split partials of each (row, head) by log-sum-exp.
template <int DV>
__global__ void __launch_bounds__(256) lse_merge(AttnArgs a) {
    const sa_problem& p = a.p;
    const int S = a.splits;
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, head)
    const long total = (long)p.B * p.n_q * p.Hq;
    if (item >= total) return;
    const int lane = threadIdx.x & 63;
    const long row = item / p.Hq;
    const int head = (int)(item % p.Hq);
    const int b = (int)(row / p.n_q), i = (int)(row % p.n_q);
    // partial s holds m_s, l_s and o_s / l_s; weight w_s = l_s 2^(m_s - M)
    const float* part = static_cast<const float*>(a.partial);
    const float* ml = part + item * S * 2;
    const uint16_t* po = partial_o(part, total * S) + item * (int64_t)S * DV;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
    float l = 0.f;
    constexpr int PER = DV / 64;
    static_assert(PER == 8, "one 16-byte load per lane and split");
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            const float ms = ml[2 * s];
            if (ms == -INFINITY) continue;
            const float w = exp2f(ms - M) * ml[2 * s + 1];
            l += w;
            const uint4 u = *reinterpret_cast<const uint4*>(po + s * DV + lane * PER);
            const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = fmaf(w, bf16_lo(uw[e]), o[2 * e]);
                o[2 * e + 1] = fmaf(w, bf16_hi(uw[e]), o[2 * e + 1]);
            }
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = static_cast<uint16_t*>(a.O.data) + b * a.O.s0 + head * a.O.s1 + (int64_t)i * a.O.s2 + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = f32_to_bf16_rne(o[e] * inv);
    if (a.lse && lane == 0) a.lse[b * a.lse_bs + (int64_t)head * p.n_q + i] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------- attn_mla_lds
// Latent-head attention for 32-head groups (Hq/Hkv a multiple of 32, V = the first d_v
// columns of K).  One workgroup per (query row, candidate split); wave w owns query heads
// 32w..32w+31.  Gathered rows reach LDS through buffer loads that write LDS directly
// (no staging registers), in a ring of four 32-row tiles: while tiles t and t + 1 are read,
// t + 2 and t + 3 are in flight.  Iteration t writes the P^T fragments of tile t (computed in
// the previous iteration) to LDS, runs S^T = K Q^T of tile t + 1 (v_mfma_f32_16x16x32_bf16,
// Q^T fragments in registers), then O^T += V^T P^T of tile t (v_mfma_f32_32x32x16_bf16) with
// the softmax of tile t + 1 between those MFMAs, reading V^T out of the same row-major tile
// with transposing LDS reads (ds_read_b64_tr_b16); each wave accumulates O^T for its slice of
// the value columns over all heads, so P goes through LDS.  Each head's reference
// maximum is fixed at its first valid tile, so the accumulators are never rescaled: any
// reference gives the same softmax, and while no logit exceeds it by more than 64 (exp2
// units) every probability and sum stays far inside fp32 range.  A set that breaks this
// margin is run a second time against its true maximum, found during the first run.
namespace mla {
constexpr int T = 32;                  // rows per tile
constexpr int DQK = 576, DV = 512;
constexpr int CHR = DQK / 8;           // 16-byte chunks per row
constexpr int ROWB = DQK * 2;          // bytes per row in LDS
constexpr int TILE_B = T * ROWB;       // bytes per tile
constexpr int NI_ALL = T * CHR / 64;   // 16-byte LDS-direct loads per tile, 64 lanes each
constexpr int MAXE = 2048;             // candidates per workgroup
constexpr int RING = 4;                // tile slots in LDS
constexpr float kLazy = 64.f;          // exp2 headroom above the reference maximum
// Tile layout in LDS (36 KB): 32 main blocks of 1 KB, block 4 rg + cg holding 16-byte chunks
// 16 cg .. 16 cg + 15 of rows 4 rg .. 4 rg + 3 (row r at slot 16 (r & 3) + cslot(r, chunk % 16)),
// then 4 tail blocks at 32 KB, tail block j holding chunks 64..71 of rows 8 j .. 8 j + 7 (row r
// at slot 8 (r & 7) + ((chunk - 64) ^ tswz(r))).  One LDS-direct load fills one block from 4
// (or 8) rows, so each load reads whole 128-byte lines; the swizzles make the 16-row reads of
// the K operand and the 4-row transposing reads of the V operand free of bank conflicts.
// Row swizzle: a linear map of the row's low four bits (bit0 = r0, bit1 = r1, bit2 = r0^r1^r2,
// bit3 = r0^r3).  A 128-bit read serves half a wave at a time: the K-operand reads (16 rows x
// two adjacent chunks per half wave) and the 4-row transposing V reads then touch every bank
// once per pass.
__device__ __forceinline__ int rswz(int r) {
    return (r & 3) | (((r ^ (r >> 1) ^ (r >> 2)) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 3);
}
__device__ __forceinline__ int cslot(int r, int c) { return c ^ rswz(r); }
// chunk (0..15) of row r stored in slot y (inverse of cslot)
__device__ __forceinline__ int cslot_inv(int r, int y) { return y ^ rswz(r); }
__device__ __forceinline__ int tswz(int r) { return (r >> 1) & 7; }
}  // namespace mla


// IDX: paged pools.  The offset list holds pool row indices, and every lane of a tile load
// forms its own 64-bit address (pool base + row * row stride + column), since a pool may
// exceed the 4 GiB a buffer resource reaches; an empty slot reads the zero row instead.

template <int NW, bool IDX>
__global__ void __launch_bounds__(64 * NW) attn_mla_lds(AttnArgs a) {
    using namespace mla;
    constexpr int NI = NI_ALL / NW;    // loads per wave per tile
    static_assert(NI * NW == NI_ALL, "tile loads must split evenly over the waves");
    constexpr int MW = DV / 32 / NW;   // 32-row tiles of O^T (rows = d) owned by one wave
    static_assert(MW * NW * 32 == DV, "the value columns must split evenly over the waves");
    constexpr int PD = 2;              // k-steps of K operands read ahead of their MFMAs
    constexpr int PB = 2 * NW * 1024;  // bytes of P^T fragments per tile
    __shared__ __attribute__((aligned(16))) uint8_t ring[RING * TILE_B];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[PB];
    __shared__ uint32_t s_off[MAXE];

    const sa_problem& p = a.p;
    const int G = p.Hq / p.Hkv;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n32 = lane & 31, h = lane >> 5, l15 = lane & 15, g = lane >> 4;
    const int S = a.splits;
    // Split sets: the splits of one row run on one XCD (workgroups go round-robin over the
    // eight XCDs), so that row's query fragments come from HBM once and from L2 after
    long unit = blockIdx.x;
    if (S > 1) {
        const long units = (long)p.B * p.n_q * p.Hkv * S;
        unit = (long)(blockIdx.x % 8) * ((units + 7) / 8) + blockIdx.x / 8;
        if (unit >= units) return;
    }
    const int split = (int)(unit % S);
    const long rowkv = unit / S;
    const int hk = (int)(rowkv % p.Hkv);
    const long row = rowkv / p.Hkv;
    const int b = (int)(row / p.n_q), i = (int)(row % p.n_q);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const uint32_t rowb = (uint32_t)(a.K.s2 * 2);
    const uint32_t SENT = IDX ? (uint32_t)a.pool_rows : 0x80000000u;  // offset-list value of an empty slot

    const int per = (p.k + S - 1) / S;
    const int e_begin = split * per;
    const int ne = max(0, min(p.k, e_begin + per) - e_begin);
    const int32_t* ix = a.idx + row * (int64_t)p.k + e_begin;
    // byte offsets of the candidate rows (out-of-range offset for invalid entries, which
    // the buffer loads turn into zero rows); the number of tiles up to the last one holding
    // a valid candidate goes through the P buffer, which is first written inside the loop
    int* s_nt = reinterpret_cast<int*>(pbuf);
    if (threadIdx.x == 0) *s_nt = 0;
    // Q^T fragments (B operand of S^T): head 32 wv + 16 q + lane%16, d = 32 s + 8 (lane/16) + 0..7.
    // Issued first, then every candidate index of this thread, so that the row's input
    // latencies overlap instead of adding up.
    constexpr int KS = DQK / 32;       // k-steps of S^T on 16x16x32 fragments
    uint4 qf[KS][2];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.Q.data) + b * a.Q.s0 + (hk * G + 32 * wv + l15) * a.Q.s1 +
                             (int64_t)i * a.Q.s2 + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int q = 0; q < 2; ++q) qf[s][q] = *reinterpret_cast<const uint4*>(qp + 16 * q * a.Q.s1 + 32 * s);
    }
    constexpr int EPT = MAXE / (64 * NW);  // candidate entries per thread
    int jv[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = (int)threadIdx.x + 64 * NW * k;
        jv[k] = e < ne ? ix[e] : -1;
    }
    __syncthreads();
    const int ne64 = (ne + 63) & ~63;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = (int)threadIdx.x + 64 * NW * k;
        if (e < ne64) {  // uniform per wave (ne64 is a multiple of 64)
            const int j = jv[k];
            const int64_t row = j >= 0 && j < L ? (IDX ? kv_row(a, b, j) : (int64_t)j) : -1;
            const bool ok = row >= 0;
            s_off[e] = ok ? (IDX ? (uint32_t)row : (uint32_t)row * rowb) : SENT;
            const uint64_t bal = __ballot(ok);
            if (lane == 0 && bal != 0) atomicMax(s_nt, (e >> 5) + ((bal >> 32) != 0 ? 2 : 1));
        }
    }
    __syncthreads();
    const int nt = __builtin_amdgcn_readfirstlane(*s_nt);
    wait_vmcnt<0>();  // (already true: the loaded values were used) no load of the compiler's own is pending

    const char* kbase = static_cast<const char*>(a.K.data) + ((IDX ? 0 : b * a.K.s0) + hk * a.K.s1) * 2;
    v4i krs;
    krs[0] = (int)(uint32_t)(uintptr_t)kbase;
    krs[1] = (int)(uint32_t)((uintptr_t)kbase >> 32);
    krs[2] = (int)((int64_t)p.n_kv * rowb);  // (unused by the paged variant)
    krs[3] = 0x00020000;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
    // Loads of one tile by this wave: main blocks wv NM .. wv NM + NM - 1 (rows 4 (block / 4) +
    // lane / 16), then tail blocks wv NT .. wv NT + NT - 1 (rows 8 j + lane / 8).
    constexpr int NM = 32 / NW, NT = 4 / NW, NRG = NM / 4;
    // Buffer offsets of this lane's rows of tile `tile`.  Tiles at or past nt get an
    // out-of-range offset: their loads move no data and only write zeros into a free ring
    // slot, which keeps the count of loads per tile constant.
    struct TileOff { uint32_t m[NRG], t[NT]; };
    auto tile_offsets = [&](int tile) {
        TileOff o;
        const bool real = tile < nt;
        const uint32_t* off = s_off + min(tile, nt - 1) * T;  // read unconditionally (no branch)
#pragma unroll
        for (int q = 0; q < NRG; ++q) {
            const int r = 4 * (wv * NRG + q) + (lane >> 4);
            const uint32_t v = off[r];
            o.m[q] = real ? (IDX ? v : v + 16u * (uint32_t)cslot_inv(r, lane & 15)) : SENT;
        }
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int r = 8 * (wv * NT + q) + (lane >> 3);
            const uint32_t v = off[r];
            o.t[q] = real ? (IDX ? v : v + 16u * (uint32_t)(64 + ((lane & 7) ^ tswz(r)))) : SENT;
        }
        return o;
    };
    auto dma = [&](int tile, int ii, const TileOff& o) {
        const uint32_t base = ring_lds + (uint32_t)((tile % RING) * TILE_B);
        if (ii < NM) {
            const int blk = wv * NM + ii;
            if (IDX) {
                const int r = 4 * (wv * NRG + (ii >> 2)) + (lane >> 4);
                const uint32_t col = 16u * (uint32_t)cslot_inv(r, lane & 15) + 256u * (uint32_t)(ii & 3);
                const uint32_t row = o.m[ii >> 2];
                lds_dma16_g(base + 1024u * (uint32_t)blk,
                            (row == SENT ? reinterpret_cast<const char*>(kZeroRow) : kbase + (uint64_t)row * rowb) + col);
            } else {
                lds_dma16(krs, base + 1024u * (uint32_t)blk, o.m[ii >> 2], 256u * (uint32_t)(ii & 3));
            }
        } else {
            const int j = wv * NT + (ii - NM);
            if (IDX) {
                const int r = 8 * j + (lane >> 3);
                const uint32_t col = 16u * (uint32_t)(64 + ((lane & 7) ^ tswz(r)));
                const uint32_t row = o.t[ii - NM];
                lds_dma16_g(base + 32768u + 1024u * (uint32_t)j,
                            (row == SENT ? reinterpret_cast<const char*>(kZeroRow) : kbase + (uint64_t)row * rowb) + col);
            } else {
                lds_dma16(krs, base + 32768u + 1024u * (uint32_t)j, o.t[ii - NM], 0u);
            }
        }
    };

    // K operand of S^T k-step s, position tile pt: row r = 16 pt + lane%16, chunk c = 4 s + lane/16;
    // kadr[pt][s % 4] + 1024 (s / 4) for s < 16, tail blocks for s = 16, 17
    // (row 16 + r has the swizzles of row r, so position tile 1 sits at a fixed offset:
    // 16 KB in the main blocks, 2 KB in the tail blocks)
    int kadr[4], ktail[2];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) kadr[k4] = 4096 * (l15 >> 2) + 256 * (l15 & 3) + 16 * cslot(l15, 4 * k4 + g);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
        ktail[k2] = 32768 + 1024 * (l15 >> 3) + 16 * (8 * (l15 & 7) + ((4 * k2 + g) ^ tswz(l15)));
    // V operand of O^T (transposing reads): this lane supplies row r = 16 s' + 8 h + 4 e2 + lane%16/4
    // and 8 bytes of chunk 4 mt + c2, c2 = 2 (lane/16 % 2) + lane%4/2.  The chunk's slot splits
    // into bits 0-1 (lane constant) and bits 2-3 = mt % 4 ^ (swizzle bits 2-3): address
    // vlo[e2] + ((64 (mt % 4)) ^ vx[e2]) + 1024 (mt / 4) + 16384 s'
    const int g2 = (lane >> 4) & 1, vc2 = 2 * g2 + ((l15 >> 1) & 1);
    int vlo[2], vx[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int r = 8 * h + 4 * e2 + (l15 >> 2);
        const int X = rswz(r);
        vlo[e2] = 4096 * (r >> 2) + 256 * (r & 3) + 16 * (vc2 ^ (X & 3)) + 8 * (l15 & 1);
        vx[e2] = 16 * (X & 12);
    }
    // P^T fragment of head group grp, k-step s' (positions 16 s' + 8 h + 0..7): 16 bytes at
    // ((s' NW + grp) 2 + h) 512 + 16 n32 of the P buffer
    const int pread = 16 * (32 * h + n32);
    uint8_t* const pw = pbuf + (size_t)(((g >> 1) * 32) * 16 + 8 * (g & 1));

    f32x16 oacc[MW][NW];
#pragma unroll
    for (int t2 = 0; t2 < MW; ++t2)
#pragma unroll
        for (int gr = 0; gr < NW; ++gr)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[t2][gr][e] = 0.f;
    // softmax state per head group q: fixed reference (log2 units; 0 until the first tile
    // with a valid candidate), the raw-logit level above which a probability would leave the
    // fp32 headroom, this lane's largest raw logit and exp-sum
    float m_ref[2] = {0.f, 0.f}, thr[2], m_lane[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
    bool ref_set = false;
    const float sl2 = a.scale * kLog2e;
    thr[0] = thr[1] = kLazy / sl2;

    // S^T = K Q^T of the tile in ring slot kt: acc[pt][q] holds S^T[pos 16 pt + 4 (lane/16) + r]
    // [head 16 q + lane%16]; step(s) runs once after the MFMAs of k-step s (loads of a later
    // tile, softmax work of the previous tile)
    constexpr int VPM = 1;  // vector-ALU instructions placed after each MFMA of S^T
    auto s_tile = [&](const uint8_t* kt, f32x4 (&acc)[2][2], auto step) {
        auto kread = [&](int s, int pt) {
            const int a_ = s < 16 ? kadr[s & 3] + 1024 * (s >> 2) + 16384 * pt : ktail[s - 16] + 2048 * pt;
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kt + a_));
        };
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[pt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kb[PD][2];
#pragma unroll
        for (int s = 0; s < PD; ++s)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) kb[s][pt] = kread(s, pt);
        // Each k-step is its own scheduling region (sched_barrier), so the reads for k-step
        // s + PD stay ahead of the MFMAs of k-step s instead of sinking next to their use.
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 c0 = kb[s % PD][0], c1 = kb[s % PD][1];
            if (s + PD < KS) {
                kb[s % PD][0] = kread(s + PD, 0);
                kb[s % PD][1] = kread(s + PD, 1);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bf16x8 qb = __builtin_bit_cast(bf16x8, qf[s][q]);
                acc[0][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c0, qb, acc[0][q], 0, 0, 0);
                acc[1][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c1, qb, acc[1][q], 0, 0, 0);
            }
            step(s);
            if (s + PD < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    f32x4 sacc[2][2];
    // Softmax numerators of the S^T tile in sacc (raw logits; masked positions already -inf)
    // against the fixed reference, in parts that the O^T MFMAs of the previous tile cover:
    // parts 0-1 the largest raw logit of head group q and the headroom check, parts 2-5 the
    // exponentials of one (position tile, head group) each.  The bf16 P^T fragments stay in
    // registers (pk) until the next iteration writes them to the P buffer.
    bool over = false;
    uint32_t pk[2][2][2];
    auto soft_part = [&](int part) {
        if (part < 2) {
            const int q = part;
            const f32x4 &u = sacc[0][q], &v = sacc[1][q];
            const float mx = fmaxf(fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3])), fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
            m_lane[q] = fmaxf(m_lane[q], mx);
            over |= mx > thr[q];
        } else if (part < 6) {
            const int pt = (part - 2) >> 1, q = (part - 2) & 1;
            // v_exp_f32 directly: results below 2^-126 of the reference flush to zero, masked
            // positions (-inf) give exactly 0
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(fmaf(sacc[pt][q][r], sl2, -m_ref[q]));
            lsum[q] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
            const bf16x2 p01 = {(__bf16)pv[0], (__bf16)pv[1]}, p23 = {(__bf16)pv[2], (__bf16)pv[3]};
            pk[pt][q][0] = __builtin_bit_cast(uint32_t, p01);
            pk[pt][q][1] = __builtin_bit_cast(uint32_t, p23);
        }
    };
    // invalid positions of the S^T tile in sacc (zero rows) get -inf logits; the first tile
    // with a valid candidate fixes each head's reference maximum (both rare: uniform branches)
    auto prep = [&](uint32_t msk) {
        if (msk != 0xffffffffu) {
            const uint32_t mg = msk >> (4 * g);
#pragma unroll
            for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (!((mg >> (16 * pt + r)) & 1u)) sacc[pt][q][r] = -INFINITY;
        }
        if (!ref_set && msk != 0u) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const f32x4 &u = sacc[0][q], &v = sacc[1][q];
                const float mx = fmaxf(fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3])), fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
                m_ref[q] = colmax4(mx) * sl2;
                thr[q] = (m_ref[q] + kLazy) / sl2;
            }
            ref_set = true;
        }
    };
    // validity of tile u: tile_off(u) reads position 32 u + lane % 32 of the offset list and
    // valid_mask turns it into bit n = position 32 u + n holds a valid candidate.  Lane % 32
    // comes from the lane mask, recomputed here (volatile: kept at its place) so that no
    // long-lived register holds this address (a spilled one would be reloaded before the tile
    // loop, and the wait for it would stall every iteration on the tile loads).
    auto tile_off = [&](int u) {
        uint32_t l32;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0" : "=v"(l32));
        return s_off[T * u + (l32 & 31u)];
    };
    auto valid_mask = [SENT](uint32_t off) { return (uint32_t)__ballot(off != SENT); };
    // P^T fragments of the last softmax into the P buffer
    auto put_p = [&]() {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *reinterpret_cast<uint2*>(pw + ((pt * NW + wv) * 2) * 512 + 16 * (16 * q + l15)) = make_uint2(pk[pt][q][0], pk[pt][q][1]);
    };
    // O^T[d slice of this wave][all heads] += V^T P^T for the tile in ring slot tb
    constexpr int VPO = 4;  // vector-ALU instructions placed after each MFMA of O^T
    auto o_tile = [&](const uint8_t* tb, auto step) {
        const uint8_t* pr = pbuf + pread;
        auto vread = [&](int s2, int t2) {
            const int mt = MW * wv + t2;
            const uint8_t* vb = tb + 1024 * (mt >> 2) + 16384 * s2;
            return __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lds_tr_read(vb + vlo[0] + ((64 * (mt & 3)) ^ vx[0])),
                                                lds_tr_read(vb + vlo[1] + ((64 * (mt & 3)) ^ vx[1])), 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 pf[NW];
#pragma unroll
        for (int gr = 0; gr < NW; ++gr)
            pf[gr] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pr + (gr * 2) * 512));
        bf16x8 va = vread(0, 0);
#pragma unroll
        for (int st = 0; st < 2 * MW; ++st) {
            const int t2 = st % MW;
            const bf16x8 vc = va;
            if (st + 1 < 2 * MW) va = vread((st + 1) / MW, (st + 1) % MW);
#pragma unroll
            for (int gr = 0; gr < NW; ++gr) {
                oacc[t2][gr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, pf[gr], oacc[t2][gr], 0, 0, 0);
                // P^T of the second k-step replaces each fragment right after its last use
                if (st == MW - 1)
                    pf[gr] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pr + ((NW + gr) * 2) * 512));
            }
            step(st);
            // each step its own scheduling region: the reads first, then every MFMA followed
            // by a few of the step's vector-ALU instructions
            if (st + 1 < 2 * MW) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int gr = 0; gr < NW; ++gr) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, VPO, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    for (int pass = 0; pass < 2; ++pass) {
    over = false;
    // from here on the waits count tile loads only
    if (nt > 0) {
#pragma unroll
        for (int tile = 0; tile < RING - 1; ++tile) {
            const TileOff o = tile_offsets(tile);
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) dma(tile, ii, o);
        }
        wait_vmcnt<((RING - 2) * NI < 63 ? (RING - 2) * NI : 63)>();  // (at least) tile 0 has landed
        tile_barrier();
        s_tile(ring, sacc, [&](int) {});
        prep(valid_mask(tile_off(0)));
#pragma unroll
        for (int part = 0; part < 6; ++part) soft_part(part);
    }
    // Iteration t: P^T of tile t (computed in the previous iteration) to the P buffer, S^T of
    // tile t + 1, then O^T of tile t with the softmax of tile t + 1 between its MFMAs.  Ring
    // slots: t (V of O^T), t + 1 (K of S^T), t + 2 and t + 3 in flight.
    for (int t = 0; t < nt; ++t) {
        wait_vmcnt<(RING - 3) * NI>();  // tile t + 1 has landed; only tile t + 2 may still be in flight
        tile_barrier();                 // every wave is past O^T of tile t - 1: its slot and P are free
        put_p();
        // validity of tile t + 1 (past the last tile: nothing valid, its softmax is discarded)
        const uint32_t offn = tile_off(min(t + 1, nt - 1));
        const TileOff dof = tile_offsets(t + RING - 1);
        // S^T of tile t + 1 (zero rows when t + 1 = nt: computed and discarded, which keeps the
        // loop body free of branches)
        s_tile(ring + ((t + 1) % RING) * TILE_B, sacc, [&](int s) {
#pragma unroll
            for (int ii = 0; ii < NI; ++ii)
                if ((ii * KS) / NI == s) dma(t + RING - 1, ii, dof);
        });
        prep(t + 1 < nt ? valid_mask(offn) : 0u);
        wait_lgkmcnt0();
        tile_barrier();
        o_tile(ring + (t % RING) * TILE_B, [&](int st) { soft_part(st); });
    }
    // the last tiles' loads (zero rows past nt) land before the ring is reused
    wait_vmcnt<0>();
    __syncthreads();
    int* s_over = reinterpret_cast<int*>(ring);
    if (threadIdx.x == 0) *s_over = 0;
    __syncthreads();
    if (over) *s_over = 1;
    __syncthreads();
    const bool again = *s_over != 0;
    __syncthreads();
    if (!again) break;
    // a probability left fp32 headroom: run the set again against the true maximum
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        m_ref[q] = colmax4(m_lane[q]) * sl2;
        thr[q] = (m_ref[q] + kLazy) / sl2;
        lsum[q] = 0.f;
    }
#pragma unroll
    for (int t2 = 0; t2 < MW; ++t2)
#pragma unroll
        for (int gr = 0; gr < NW; ++gr)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[t2][gr][e] = 0.f;
    }
    // per-head reference and exp-sum (lanes with the same lane%16 hold disjoint positions),
    // kept in the last ring slot, which the output staging below does not reach
    float* s_ml = reinterpret_cast<float*>(ring + (RING - 1) * TILE_B);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        lsum[q] += __shfl_xor(lsum[q], 16);
        lsum[q] += __shfl_xor(lsum[q], 32);
        if (g == 0) {
            s_ml[32 * wv + 16 * q + l15] = lsum[q] > 0.f ? m_ref[q] : -INFINITY;
            s_ml[32 * NW + 32 * wv + 16 * q + l15] = lsum[q];
        }
    }
    __syncthreads();
    if (S == 1 && a.lse && g == 0) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            a.lse[b * a.lse_bs + (int64_t)(hk * G + 32 * wv + 16 * q + l15) * p.n_q + i] =
                lsum[q] > 0.f ? (m_ref[q] + log2f(lsum[q])) * kLn2 : -INFINITY;
    }
    // lane holds O^T[d = 32 (MW wv + t2) + 8 (e/4) + 4 h + e%4][head 32 gr + n32]
    if (S == 1) {
        // Stage bf16 rows of O in LDS (the ring is free now; each wave owns a region and
        // handles GR head groups per round) and store them as whole row pieces.
        constexpr int GR = NW < 2 ? NW : 2;  // head groups per round
        constexpr int OP = MW * 64 + 8;      // LDS pitch of one staged head row (bytes)
        constexpr int LPR = MW * 64 / 16;    // lanes per staged row
        uint8_t* stg = ring + wv * (32 * GR * OP);
#pragma unroll
        for (int r0 = 0; r0 < NW; r0 += GR) {
#pragma unroll
            for (int gq = 0; gq < GR; ++gq) {
                const float l = s_ml[32 * NW + 32 * (r0 + gq) + n32];
                const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
                for (int t2 = 0; t2 < MW; ++t2)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x16& o = oacc[t2][r0 + gq];
                        const bf16x2 v01 = {(__bf16)(o[4 * q] * inv), (__bf16)(o[4 * q + 1] * inv)};
                        const bf16x2 v23 = {(__bf16)(o[4 * q + 2] * inv), (__bf16)(o[4 * q + 3] * inv)};
                        *reinterpret_cast<uint2*>(stg + (32 * gq + n32) * OP + 2 * (32 * t2 + 8 * q + 4 * h)) =
                            make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
                    }
            }
            wait_lgkmcnt0();  // this wave reads back only what it wrote
#pragma unroll
            for (int rr = 0; rr < 32 * GR; rr += 64 / LPR) {
                const int hr = rr + lane / LPR, j = lane % LPR;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + hr * OP + 16 * j);
                uint16_t* op = static_cast<uint16_t*>(a.O.data) + b * a.O.s0 + (hk * G + 32 * r0 + hr) * a.O.s1 +
                               (int64_t)i * a.O.s2 + 32 * MW * wv + 8 * j;
                *reinterpret_cast<uint4*>(op) = v;
            }
            wait_lgkmcnt0();
        }
    } else {
        // partial in MFMA fragment order: fragment f = mt NW + gr of (row, hk, split) holds
        // 64 lanes x 16 values of o / l, 32 contiguous bytes per lane
        float* part = static_cast<float*>(a.partial);
        const int64_t slots = (int64_t)p.B * p.n_q * p.Hq * S;
        uint16_t* pbase = partial_o(part, slots) + ((rowkv * S + split) * (int64_t)G) * DV;
#pragma unroll
        for (int gr = 0; gr < NW; ++gr) {
            const float l = s_ml[32 * NW + 32 * gr + n32];
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int t2 = 0; t2 < MW; ++t2) {
                const f32x16& o = oacc[t2][gr];
                uint32_t w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bf16x2 v = {(__bf16)(o[2 * e] * inv), (__bf16)(o[2 * e + 1] * inv)};
                    w[e] = __builtin_bit_cast(uint32_t, v);
                }
                uint4* dst = reinterpret_cast<uint4*>(pbase + ((MW * wv + t2) * NW + gr) * 1024 + lane * 16);
                dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
                dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            }
            if (wv == 0 && h == 0) {
                float* ml = part + ((row * p.Hq + hk * G + 32 * gr + n32) * (int64_t)S + split) * 2;
                ml[0] = s_ml[32 * gr + n32];
                ml[1] = s_ml[32 * NW + 32 * gr + n32];
            }
        }
    }
}

// Merge the split partials of attn_mla_lds (fragment order, see above): one wave per
// (row, key/value head, fragment).  Output O[head][d] from o = sum_s w_s o_s / sum_s w_s,
// w_s = l_s 2^(m_s - M), and the log-sum-exp per head.
__global__ void __launch_bounds__(256) lse_merge_frag(AttnArgs a) {
    const sa_problem& p = a.p;
    const int S = a.splits, G = p.Hq / p.Hkv, NW = G / 32, NF = (512 / 32) * NW;
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, hk, fragment)
    const long total = (long)p.B * p.n_q * p.Hkv * NF;
    if (item >= total) return;
    const int lane = threadIdx.x & 63, n32 = lane & 31, h = lane >> 5;
    const int f = (int)(item % NF);
    const long rowkv = item / NF;
    const int hk = (int)(rowkv % p.Hkv);
    const long row = rowkv / p.Hkv;
    const int b = (int)(row / p.n_q), i = (int)(row % p.n_q);
    const int mt = f / NW, gr = f % NW;
    const int head = hk * G + 32 * gr + n32;
    const float* part = static_cast<const float*>(a.partial);
    const int64_t slots = (int64_t)p.B * p.n_q * p.Hq * S;
    const float* ml = part + (row * p.Hq + head) * (int64_t)S * 2;
    const uint16_t* pb = partial_o(part, slots) + (rowkv * S) * (int64_t)G * 512 + f * 1024 + lane * 16;
    // running log-sum-exp over the splits, so that no load waits for a value computed from
    // another load; a split without valid candidates has m = -inf, l = 0 and zero o
    float M = -INFINITY, l = 0.f, o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
        const float ms = ml[2 * s], ls = ml[2 * s + 1];
        const uint4* src = reinterpret_cast<const uint4*>(pb + s * (int64_t)G * 512);
        const uint4 u0 = src[0], u1 = src[1];
        const float Mn = fmaxf(M, ms);
        const float c = M == -INFINITY ? 0.f : exp2f(M - Mn);   // rescale of what is merged so far
        const float w = ms == -INFINITY ? 0.f : exp2f(ms - Mn) * ls;
        M = Mn;
        l = l * c + w;
        const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[2 * e] = fmaf(w, bf16_lo(uw[e]), o[2 * e] * c);
            o[2 * e + 1] = fmaf(w, bf16_hi(uw[e]), o[2 * e + 1] * c);
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = static_cast<uint16_t*>(a.O.data) + b * a.O.s0 + head * a.O.s1 + (int64_t)i * a.O.s2 + 32 * mt + 4 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[4 * q] * inv) | ((uint32_t)f32_to_bf16_rne(o[4 * q + 1] * inv) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[4 * q + 2] * inv) | ((uint32_t)f32_to_bf16_rne(o[4 * q + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + 8 * q) = make_uint2(lo, hi);
    }
    if (a.lse && mt == 0 && h == 0)
        a.lse[b * a.lse_bs + (int64_t)head * p.n_q + i] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
}

template <typename T, int LPR>
hipError_t launch_rows_g(const AttnArgs& a, int G, unsigned blocks, hipStream_t s) {
    if (G == 1) hipLaunchKernelGGL((attn_rows<T, LPR, 1>), dim3(blocks), dim3(256), 0, s, a);
    else if (G == 2) hipLaunchKernelGGL((attn_rows<T, LPR, 2>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_rows<T, LPR, 4>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// The LDS-direct latent kernel: 32, 64 or 128 heads per key/value head, V aliasing the first d_v columns of K,
// 16-byte aligned rows, 32-bit row offsets and at most mla::MAXE candidates per split.
static bool mla_lds_ok(const AttnArgs& a) {
    const sa_problem& p = a.p;
    const int G = p.Hq / p.Hkv;
    const bool alias = a.V.data == a.K.data && a.V.s0 == a.K.s0 && a.V.s1 == a.K.s1 && a.V.s2 == a.K.s2;
    const long per = (p.k + a.splits - 1) / a.splits;
    // contiguous: 32-bit byte offsets into one batch's rows; paged: 32-bit row indices (the
    // value pool_rows marks an empty slot) and rows no longer than the zero row
    const bool addr = a.block_table ? (a.pool_rows < 0xffffffffLL && a.K.s2 * 2 <= kZeroRowBytes)
                                    : (int64_t)p.n_kv * a.K.s2 * 2 < (1LL << 31);
    return (G == 32 || G == 64 || G == 128) && alias && a.K.s2 % 8 == 0 && ((uintptr_t)a.K.data & 15) == 0 && addr &&
           per <= mla::MAXE;
}

// The bf16 MHA kernel: rows below 2^24 and row strides below 2^24 bytes (24-bit multiplies),
// every head's slice of K and V below 2^31 bytes, candidate lists read four at a time.
static bool rows_buf_ok(const AttnArgs& a) {
    const sa_problem& p = a.p;
    const int64_t rows = a.block_table ? a.pool_rows : (int64_t)p.n_kv;
    return a.Q.dtype == SA_BF16 && p.Hq == p.Hkv && p.d_qk == p.d_v && (p.d_qk == 64 || p.d_qk == 128 || p.d_qk == 256) &&
           (p.k % 4 == 0) && rows * a.K.s2 * 2 < (1LL << 31) && rows * a.V.s2 * 2 < (1LL << 31) &&
           ((uintptr_t)a.idx & 15) == 0 && rows < (1 << 24) && a.K.s2 * 2 < (1 << 24) && a.V.s2 * 2 < (1 << 24);
}

// The tile kernel: bf16 MHA with d = 128, at least 64 query rows, a history of at most
// tile::MAXN positions, and budgets large enough that a block's selections cover most key
// tiles (64 rows x k >= 2 n_kv); candidate lists read four at a time.
static bool tile_shape_ok(const sa_problem& p) {
    return p.Hq == p.Hkv && p.d_qk == tile::D && p.d_v == tile::D && p.n_kv <= tile::MAXN && p.n_q >= 64 &&
           p.k % 4 == 0 && (int64_t)p.k * 64 >= 2LL * p.n_kv;
}
static bool tile_ok(const AttnArgs& a) {
    return a.Q.dtype == SA_BF16 && tile_shape_ok(a.p) && ((uintptr_t)a.idx & 15) == 0;
}
// workspace of the tile kernel: the rows' selection bitmaps, then the row blocks' tile lists
static size_t tile_bits_bytes(const sa_problem& p) {
    return ((size_t)p.B * p.n_q * (tile::MAXN / 8) + 255) & ~(size_t)255;
}
static size_t tile_ws_bytes(const sa_problem& p) {
    const size_t nsb = (size_t)(p.n_q + tile::SUB - 1) / tile::SUB;
    return tile_bits_bytes(p) + (size_t)p.B * nsb * tile::LIST * sizeof(int32_t);
}

bool attn_paged_ok(const AttnArgs& a) {
    return attn_uses_mla(a.p, a.Q.dtype) ? mla_lds_ok(a) : (tile_ok(a) || rows_buf_ok(a));
}

// one workgroup per query row; the row's history as a bitmap in LDS marks the positions seen
__global__ void __launch_bounds__(256) check_indices(sa_problem p, const int32_t* idx, Status* status, int repeats) {
    extern __shared__ uint32_t seen[];
    const long row = blockIdx.x;
    const int b = (int)(row / p.n_q), i = (int)(row % p.n_q);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    if (repeats)
        for (int w = threadIdx.x; w < (p.n_kv + 31) >> 5; w += 256) seen[w] = 0u;
    __syncthreads();
    bool bad = false;
    const int32_t* ix = idx + row * (int64_t)p.k;
    for (int e = threadIdx.x; e < p.k; e += 256) {
        const int j = ix[e];
        if (j == -1) continue;
        if (j < 0 || j >= L) {
            bad = true;
            continue;
        }
        if (repeats) {
            const uint32_t bit = 1u << (j & 31);
            if (atomicOr(&seen[j >> 5], bit) & bit) bad = true;
        }
    }
    if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(&status->flags, 1u << SA_ERR_INDEX);
}

bool attn_uses_mla(const sa_problem& p, int dtype) {
    const int G = p.Hq / p.Hkv;
    return dtype == SA_BF16 && G % 16 == 0 && G <= 128 && p.d_qk == 576 && p.d_v == 512;
}

int attn_splits(const sa_problem& p) {
    // about one workgroup per CU, at least 4 tiles of candidates per split, and at most
    // mla::MAXE candidates per workgroup; SA_SPLITS overrides the first two (at least one
    // tile per split)
    const long units = (long)p.B * p.n_q * p.Hkv;
    long s = (256 + units - 1) / units;
    long cap = p.k / (4 * kTile);
    if (cap < 1) cap = 1;
    if (s > cap) s = cap;
    const int forced = env_int("SA_SPLITS", 0);
    if (forced > 0) s = std::min<long>(forced, std::max<long>(1, (p.k + kTile - 1) / kTile));
    const long need = (p.k + mla::MAXE - 1) / mla::MAXE;
    if (s < need) s = need;
    if (s < 1) s = 1;
    return (int)s;
}

hipError_t launch_check_indices(const sa_problem& p, const int32_t* idx, Status* status, hipStream_t s) {
    const int repeats = p.n_kv <= kCheckMaxPositions;
    const size_t lds = repeats ? (size_t)((p.n_kv + 31) >> 5) * sizeof(uint32_t) : 0;
    hipLaunchKernelGGL(check_indices, dim3((unsigned)((long)p.B * p.n_q)), dim3(256), lds, s, p, idx, status, repeats);
    return hipGetLastError();
}

size_t attn_partial_bytes(const sa_problem& p) {
    // the tile kernel's selection bitmaps and tile lists, or the latent kernel's split partials
    const size_t tile = tile_shape_ok(p) ? tile_ws_bytes(p) : 0;
    const int S = attn_splits(p);
    if (S <= 1) return tile;
    // (m, l) in fp32 and o / l in bf16 per (row, head, split), the o block 256-byte aligned
    const size_t slots = (size_t)p.B * p.n_q * p.Hq * S;
    const size_t part = ((slots * 8 + 255) & ~(size_t)255) + slots * (size_t)p.d_v * sizeof(uint16_t);
    return part > tile ? part : tile;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
    const sa_problem& p = a.p;
    if (a.block_table && !attn_paged_ok(a)) return hipErrorInvalidValue;  // only the two kernels above translate pages
    if (attn_uses_mla(p, a.Q.dtype)) {
        const int G = p.Hq / p.Hkv;
        const long units = (long)p.B * p.n_q * p.Hkv * a.splits;
        const bool lds_kernel = mla_lds_ok(a);
        if (lds_kernel) {
            const dim3 grid((unsigned)(a.splits > 1 ? 8 * ((units + 7) / 8) : units));
            if (a.block_table) {
                if (G == 128) hipLaunchKernelGGL((attn_mla_lds<4, true>), grid, dim3(256), 0, s, a);
                else if (G == 64) hipLaunchKernelGGL((attn_mla_lds<2, true>), grid, dim3(128), 0, s, a);
                else hipLaunchKernelGGL((attn_mla_lds<1, true>), grid, dim3(64), 0, s, a);
            } else {
                if (G == 128) hipLaunchKernelGGL((attn_mla_lds<4, false>), grid, dim3(256), 0, s, a);
                else if (G == 64) hipLaunchKernelGGL((attn_mla_lds<2, false>), grid, dim3(128), 0, s, a);
                else hipLaunchKernelGGL((attn_mla_lds<1, false>), grid, dim3(64), 0, s, a);
            }
        } else {
            hipLaunchKernelGGL((attn_mla<576, 512>), dim3((unsigned)units), dim3(64 * (G / 16)), 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.splits == 1) return e;
        const long items = (long)p.B * p.n_q * p.Hq;
        if (lds_kernel) {
            const long frags = (long)p.B * p.n_q * p.Hkv * (512 / 32) * (G / 32);
            hipLaunchKernelGGL(lse_merge_frag, dim3((unsigned)((frags + 3) / 4)), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((lse_merge<512>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, a);
        }
        return hipGetLastError();
    }
    const int G = p.Hq / p.Hkv;
    if (tile_ok(a)) {
        // selections once per (batch, row block), then every head's tiles
        const long nqb = (p.n_q + tile::QR - 1) / tile::QR;
        uint32_t* gbits = static_cast<uint32_t*>(a.partial);
        int32_t* glist = reinterpret_cast<int32_t*>(static_cast<char*>(a.partial) + tile_bits_bytes(p));
        const long nsb = (p.n_q + tile::SUB - 1) / tile::SUB;
        hipLaunchKernelGGL(tile_bits, dim3((unsigned)(p.B * nsb)), dim3(1024), 0, s, a, gbits, glist);
        // pages shorter than a tile: each row's pool row is looked up on its own
        if (a.block_table && a.page_shift < 6)
            hipLaunchKernelGGL(attn_tile<true>, dim3((unsigned)(p.B * nqb * p.Hkv)), dim3(64 * tile::NWV), 0, s, a, gbits, glist);
        else
            hipLaunchKernelGGL(attn_tile<false>, dim3((unsigned)(p.B * nqb * p.Hkv)), dim3(64 * tile::NWV), 0, s, a, gbits, glist);
        return hipGetLastError();
    }
    if (a.Q.dtype == SA_BF16 && G == 1 && p.d_qk == p.d_v && (p.d_qk == 64 || p.d_qk == 128 || p.d_qk == 256)) {
        if (rows_buf_ok(a)) {
            const unsigned nblk = (unsigned)((long)p.B * ((p.n_q + 3) / 4) * p.Hkv);
            if (a.block_table) {
                // translate once into the workspace, then read pool rows
                int32_t* rows = static_cast<int32_t*>(a.partial);
                const long n = (long)p.B * p.n_q * p.k;
                hipLaunchKernelGGL(page_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, rows);
                AttnArgs t = a;
                t.idx = rows;
                if (p.d_qk == 64) hipLaunchKernelGGL((attn_rows_buf<64, true>), dim3(nblk), dim3(256), 0, s, t);
                else if (p.d_qk == 128) hipLaunchKernelGGL((attn_rows_buf<128, true>), dim3(nblk), dim3(256), 0, s, t);
                else hipLaunchKernelGGL((attn_rows_buf<256, true>), dim3(nblk), dim3(256), 0, s, t);
            } else {
                if (p.d_qk == 64) hipLaunchKernelGGL((attn_rows_buf<64, false>), dim3(nblk), dim3(256), 0, s, a);
                else if (p.d_qk == 128) hipLaunchKernelGGL((attn_rows_buf<128, false>), dim3(nblk), dim3(256), 0, s, a);
                else hipLaunchKernelGGL((attn_rows_buf<256, false>), dim3(nblk), dim3(256), 0, s, a);
            }
            return hipGetLastError();
        }
    }
    const int esz = a.Q.dtype == SA_F32 ? 4 : 2;
    const int LPR = p.d_qk * esz / 16;
    const unsigned blocks = (unsigned)((long)p.B * ((p.n_q + 3) / 4) * p.Hkv);
    if (a.Q.dtype == SA_F32) {
        if (LPR == 8) return launch_rows_g<float, 8>(a, G, blocks, s);
        if (LPR == 16) return launch_rows_g<float, 16>(a, G, blocks, s);
        return launch_rows_g<float, 32>(a, G, blocks, s);
    }
    if (LPR == 8) return launch_rows_g<uint16_t, 8>(a, G, blocks, s);
    if (LPR == 16) return launch_rows_g<uint16_t, 16>(a, G, blocks, s);
    return launch_rows_g<uint16_t, 32>(a, G, blocks, s);
}

}  // namespace sa
