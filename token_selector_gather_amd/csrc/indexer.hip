// Indexer score kernels.
//
// r[b,i,j] = sum_h w[b,i,h] * ReLU(<q_idx[b,i,h,:], k_idx[b,j,:]>)  for visible j
// ("PaperTrace 2.2 · Fine-grained indexing", §1.1 and §3.2: per-query index heads, one
// index key per token shared by all heads, query-dependent head weights).
//
// Matrix-core path (bf16 index queries; bf16 or OCP-e4m3 index keys).  The contraction
// is a GEMM with M = (query, index head) rows, N = history positions, K = d_idx, on
// v_mfma_f32_16x16x32_bf16.  One wave owns 64 rows (4 M-tiles: 64/Hidx queries) and a
// chunk of 256 positions; its index-query fragments stay in registers for the whole
// chunk.  e4m3 keys widen to bf16 exactly in hardware (v_cvt_scalef32_pk_bf16_fp8, scale
// 1).  The epilogue applies ReLU and the head weights to the fp32 accumulators and sums
// the heads inside the accumulator layout (in-lane, then xor-16 / xor-32 lane swaps), so
// the order of every reduction is the same for every position j: byte-identical keys get
// bit-identical scores.
//
// ReLU is written as (z > 0 ? z : 0*z) so that a NaN or -inf dot product stays non-finite
// and reaches the selection's finiteness check instead of being clipped to zero.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float relu_keep_nonfinite(float z) { return z > 0.f ? z : 0.f * z; }

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
    const int row = blockIdx.x;
    const int b = row / p.n_q, i = row % p.n_q;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const int j = blockIdx.y * 256 + threadIdx.x;
    float* out = a.scores + (int64_t)row * a.row_stride;
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

template <int KSTEPS, bool KE4M3>
__device__ __forceinline__ void load_b(const uint8_t* kbase_bytes, bool ok, bf16x8 (&bv)[KSTEPS], int lane) {
    const int dof = 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        if (KE4M3) {
            uint2 u = ok ? *reinterpret_cast<const uint2*>(kbase_bytes + 32 * s + dof) : make_uint2(0, 0);
            bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.x, 1.0f, false);
            bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.x, 1.0f, true);
            bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.y, 1.0f, false);
            bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u.y, 1.0f, true);
            bv[s] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        } else {
            uint4 u = ok ? *reinterpret_cast<const uint4*>(kbase_bytes + 2 * (32 * s + dof)) : make_uint4(0, 0, 0, 0);
            bv[s] = __builtin_bit_cast(bf16x8, u);
        }
    }
}

template <int KSTEPS, bool KE4M3, int H>
__global__ void __launch_bounds__(256) indexer_mfma(IndexerArgs a, int n_groups, int n_chunks) {
    const sa_problem& p = a.p;
    const int lane = threadIdx.x & 63;
    const int wave_id = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int total = p.B * n_groups * n_chunks;
    if (wave_id >= total) return;
    // longest work first: higher query groups see longer causal histories
    const int chunk = wave_id % n_chunks;
    const int rest = wave_id / n_chunks;
    const int g = n_groups - 1 - (rest % n_groups);
    const int b = rest / n_groups;
    constexpr int QPG = 64 / H;  // queries per wave group
    const int i0 = g * QPG;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};

    // visible lengths of this group's queries (lane q holds query q's length)
    int Lq = 0;
    if (lane < QPG && i0 + lane < p.n_q) Lq = visible_len(R, b, i0 + lane);
    int Lmax = Lq;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Lmax = max(Lmax, __shfl_xor(Lmax, o));

    const int j_begin = chunk * kChunk;
    const int j_end = min(j_begin + kChunk, p.n_kv);
    const int j_comp_end = min(j_end, Lmax);

    // A fragments: row r = 16*mt + lane%16 -> query r / H, head r % H; d = 32 s + 8 (lane/16)
    bf16x8 av[kMT][KSTEPS];
    float wv[kMT][4];
    if (j_begin < j_comp_end) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int r = 16 * mt + (lane & 15);
            const int qi = i0 + r / H, h = r % H;
            const bool ok = qi < p.n_q;
            const uint16_t* qb = static_cast<const uint16_t*>(a.q.data) + (ok ? (b * a.q.s0 + qi * a.q.s1 + h * a.q.s2) : 0);
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                uint4 u = ok ? *reinterpret_cast<const uint4*>(qb + 32 * s + 8 * (lane >> 4)) : make_uint4(0, 0, 0, 0);
                av[mt][s] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * mt + 4 * (lane >> 4) + e;
                const int q2 = i0 + rr / H, h2 = rr % H;
                wv[mt][e] = q2 < p.n_q ? static_cast<const float*>(a.w.data)[b * a.w.s0 + q2 * a.w.s1 + h2] : 0.f;
            }
        }
    }

    const int64_t kstride_bytes = a.k.s1 * (KE4M3 ? 1 : 2);
    const uint8_t* kb0 = static_cast<const uint8_t*>(a.k.data) + b * a.k.s0 * (KE4M3 ? 1 : 2);

    for (int j0 = j_begin; j0 < j_end; j0 += 16) {
        const int j = j0 + (lane & 15);
        if (j0 >= j_comp_end) {
            // nothing visible for any query of the group from here on
            if (a.fill_invisible && j < j_end) {
                for (int q = (lane >> 4); q < QPG; q += 4)
                    if (i0 + q < p.n_q) a.scores[(int64_t)(b * p.n_q + i0 + q) * a.row_stride + j] = -INFINITY;
            }
            continue;
        }
        bf16x8 bv[KSTEPS];
        load_b<KSTEPS, KE4M3>(kb0 + (int64_t)j * kstride_bytes, j < j_end, bv, lane);
        f32x4 acc[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][s], bv[s], acc[mt], 0, 0, 0);

        // epilogue: w * ReLU, summed over the heads of each query inside the C layout
        float part[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) t = fmaf(wv[mt][e], relu_keep_nonfinite(acc[mt][e]), t);
            part[mt] = t;
        }
        // Lane (g = lane/16) holds rows 4g..4g+3 of every M-tile.
        // H >= 16: an M-tile belongs to one query; sum tiles of the same query, then over g.
        // H == 8: rows 0-7 (g 0,1) and 8-15 (g 2,3) are two queries; sum over g pairs.
        // H == 4: each g is its own query.
        if constexpr (H >= 16) {
            constexpr int tpq = H / 16;  // tiles per query
#pragma unroll
            for (int q = 0; q < QPG; ++q) {
                float v = 0.f;
#pragma unroll
                for (int t = 0; t < tpq; ++t) v += part[q * tpq + t];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                const int qi = i0 + q;
                if (lane < 16 && qi < p.n_q) {
                    const int Lh = __shfl(Lq, q);
                    const bool vis = j < Lh;
                    if (j < j_end && (vis || a.fill_invisible))
                        a.scores[(int64_t)(b * p.n_q + qi) * a.row_stride + j] = vis ? v : -INFINITY;
                }
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                float v = part[mt];
                int qloc;
                if constexpr (H == 8) {
                    v += __shfl_xor(v, 16);
                    qloc = 2 * mt + (lane >> 5);
                } else {  // H == 4
                    qloc = 4 * mt + (lane >> 4);
                }
                const int Lh = __shfl(Lq, qloc);
                const int qi = i0 + qloc;
                const bool writer = (H == 8) ? ((lane & 16) == 0) : true;
                if (writer && qi < p.n_q) {
                    const bool vis = j < Lh;
                    if (j < j_end && (vis || a.fill_invisible))
                        a.scores[(int64_t)(b * p.n_q + qi) * a.row_stride + j] = vis ? v : -INFINITY;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
    const sa_problem& p = a.p;
    const int H = p.Hidx, D = p.d_idx;
    const bool mfma_ok = a.q.dtype == SA_BF16 && (a.k.dtype == SA_BF16 || a.k.dtype == SA_FP8_E4M3) &&
                         (H == 4 || H == 8 || H == 16 || H == 32 || H == 64) &&
                         (D == 32 || D == 64 || D == 128);
    if (mfma_ok) {
        const int n_groups = (p.n_q + (64 / H) - 1) / (64 / H);
        const int n_chunks = (p.n_kv + kChunk - 1) / kChunk;
        const long waves = (long)p.B * n_groups * n_chunks;
        const unsigned blocks = (unsigned)((waves + 3) / 4);
        const bool e4 = a.k.dtype == SA_FP8_E4M3;
#define SA_IDX_H(KS, E4, HH)                                                                               \
    if (H == HH) hipLaunchKernelGGL((indexer_mfma<KS, E4, HH>), dim3(blocks), dim3(256), 0, s, a, n_groups, n_chunks)
#define SA_IDX_KS(KS, E4) \
    do { SA_IDX_H(KS, E4, 4); SA_IDX_H(KS, E4, 8); SA_IDX_H(KS, E4, 16); SA_IDX_H(KS, E4, 32); SA_IDX_H(KS, E4, 64); } while (0)
        if (D == 32) { if (e4) SA_IDX_KS(1, true); else SA_IDX_KS(1, false); }
        else if (D == 64) { if (e4) SA_IDX_KS(2, true); else SA_IDX_KS(2, false); }
        else { if (e4) SA_IDX_KS(4, true); else SA_IDX_KS(4, false); }
#undef SA_IDX_KS
#undef SA_IDX_H
        return hipGetLastError();
    }
    dim3 grid(p.B * p.n_q, (p.n_kv + 255) / 256);
    size_t shm = sizeof(float) * ((size_t)H * D + H);
    hipLaunchKernelGGL(indexer_valu, grid, dim3(256), shm, s, a);
    return hipGetLastError();
}

}  // namespace sa
