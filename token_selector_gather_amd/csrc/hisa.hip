// Hierarchical (coarse-to-fine) selection: the small kernels around the indexer and top-k.
//
// "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the HISA paragraphs: the history is cut into
// blocks of b positions, every block is scored through a representative index key, the
// k_b best blocks are kept, and the token indexer runs only inside them, so the output is
// the same token top-k.  The scoring and the two selections reuse the indexer and top-k
// kernels on derived problems; the kernels here build those problems:
//  * block_means: representative of each complete block = the mean of its b index keys
//    (fp32 sums of the exactly decoded keys in a fixed order, divided by b, rounded once
//    to bf16);
//  * hisa_rows: number of complete blocks inside each row's visible prefix;
//  * hisa_gather: each row's candidate keys copied to a compact array, kept blocks in
//    ascending block order and then the open block [P b, L) (always a candidate), so that
//    candidate slot order is position order and the top-k tie rule carries over;
//  * hisa_map: candidate slots back to history positions.
#include "sa_internal.h"

namespace sa {
namespace {

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    // OCP e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; 0x7f / 0xff are NaN
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = e ? ldexpf(1.f + 0.125f * (float)m, (int)e - 7) : ldexpf((float)m, -9);
    if (e == 15u && m == 7u) v = __builtin_nanf("");
    return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One workgroup per (block, batch).  A key row splits into 16-byte pieces; thread (g, c)
// sums piece c over rows g, g + G, g + 2G, ... (G row groups), then the G partial sums of
// each dimension are added in group order through LDS.
constexpr int kMeanMaxD = 256;  // widest index key handled (elements)
__global__ void __launch_bounds__(256) block_means(sa_problem p, sa_tensor k, int blk, uint16_t* kbar, int es) {
    __shared__ float part[4096];  // [row group][dimension] partial sums: G * d_idx = 4096 / es
    const int B = blockIdx.x, b = blockIdx.y, nb = p.n_kv / blk;
    const int ppr = p.d_idx * es / 16, epp = 16 / es;  // pieces per row, elements per piece
    const int G = 256 / ppr;                           // row groups
    const int g = threadIdx.x / ppr, c = threadIdx.x % ppr;
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    if (g < G) {
        const uint8_t* base = static_cast<const uint8_t*>(k.data) + ((int64_t)b * k.s0 + (int64_t)B * blk * k.s1) * es + 16 * c;
        for (int t = g; t < blk; t += G) {
            const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)t * k.s1 * es);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            if (es == 1) {
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] += e4m3_value((w[e / 4] >> (8 * (e % 4))) & 0xffu);
            } else if (es == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += __uint_as_float(((w[e / 2] >> (16 * (e % 2))) & 0xffffu) << 16);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
            }
        }
        for (int e = 0; e < epp; ++e) part[g * p.d_idx + c * epp + e] = acc[e];
    }
    __syncthreads();
    for (int d = threadIdx.x; d < p.d_idx; d += 256) {
        float s = 0.f;
        for (int gg = 0; gg < G; ++gg) s += part[gg * p.d_idx + d];
        kbar[((int64_t)b * nb + B) * p.d_idx + d] = bf16_rne(s / (float)blk);
    }
}

__global__ void __launch_bounds__(256) hisa_rows(sa_problem p, int blk, int32_t* row_blk) {
    const long r = (long)blockIdx.x * 256 + threadIdx.x;
    if (r >= (long)p.B * p.n_q) return;
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    row_blk[r] = visible_len(R, (int)(r / p.n_q), (int)(r % p.n_q)) / blk;
}

// workgroup (r, s): slot s < k_blocks copies kept block s of row r, slot k_blocks the open
// block; rows are copied in 16-byte pieces
__global__ void __launch_bounds__(256) hisa_gather(sa_problem p, sa_tensor k, int blk, int k_blocks, const int32_t* bidx,
                                                   const int32_t* row_blk, uint8_t* ck, int32_t* row_tok, int es) {
    const int s = blockIdx.y;
    const long r = blockIdx.x;
    const int b = (int)(r / p.n_q), i = (int)(r % p.n_q);
    const Rows R{p.kv_len, p.q_pos0, p.n_q, p.n_kv, p.causal};
    const int L = visible_len(R, b, i);
    const int P = row_blk[r];
    const int nb = min(k_blocks, P);  // kept blocks: the first nb entries of the row's block list
    int src0, dst0, nrow;
    if (s < k_blocks) {
        if (s >= nb) return;
        src0 = bidx[r * k_blocks + s] * blk;
        dst0 = s * blk;
        nrow = blk;
    } else {
        src0 = P * blk;
        dst0 = nb * blk;
        nrow = L - P * blk;
        if (threadIdx.x == 0) row_tok[r] = nb * blk + nrow;
    }
    const int rb = p.d_idx * es, pieces = rb / 16;
    const int nc = (k_blocks + 1) * blk;
    const uint8_t* kb = static_cast<const uint8_t*>(k.data) + (int64_t)b * k.s0 * es;
    uint8_t* out = ck + (r * nc + dst0) * (int64_t)rb;
    for (int e = threadIdx.x; e < nrow * pieces; e += 256) {
        const int t = e / pieces, c = e % pieces;
        *reinterpret_cast<uint4*>(out + (int64_t)t * rb + 16 * c) =
            *reinterpret_cast<const uint4*>(kb + (int64_t)(src0 + t) * k.s1 * es + 16 * c);
    }
}

__global__ void __launch_bounds__(256) hisa_map(sa_problem p, int blk, int k_blocks, const int32_t* bidx,
                                                const int32_t* row_blk, const int32_t* cidx, int32_t* idx) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)p.B * p.n_q * p.k) return;
    const long r = e / p.k;
    const int c = cidx[e];
    if (c < 0) { idx[e] = -1; return; }
    const int P = row_blk[r], nb = min(k_blocks, P);
    idx[e] = c < nb * blk ? bidx[r * k_blocks + c / blk] * blk + c % blk : P * blk + (c - nb * blk);
}

}  // namespace

hipError_t launch_block_means(const sa_problem& p, const sa_tensor& k, int blk, uint16_t* kbar, hipStream_t s) {
    const int nb = p.n_kv / blk;
    if (nb == 0) return hipSuccess;
    const int es = k.dtype == SA_F32 ? 4 : (k.dtype == SA_BF16 ? 2 : 1);
    if (p.d_idx > kMeanMaxD || p.d_idx * es / 16 > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(block_means, dim3((unsigned)nb, (unsigned)p.B), dim3(256), 0, s, p, k, blk, kbar, es);
    return hipGetLastError();
}

hipError_t launch_hisa_rows(const sa_problem& p, int blk, int32_t* row_blk, hipStream_t s) {
    const long rows = (long)p.B * p.n_q;
    hipLaunchKernelGGL(hisa_rows, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p, blk, row_blk);
    return hipGetLastError();
}

hipError_t launch_hisa_gather(const sa_problem& p, const sa_tensor& k, int blk, int k_blocks, const int32_t* bidx,
                              const int32_t* row_blk, uint8_t* ck, int32_t* row_tok, hipStream_t s) {
    const int es = k.dtype == SA_F32 ? 4 : (k.dtype == SA_BF16 ? 2 : 1);
    hipLaunchKernelGGL(hisa_gather, dim3((unsigned)((long)p.B * p.n_q), (unsigned)(k_blocks + 1)), dim3(256), 0, s, p, k,
                       blk, k_blocks, bidx, row_blk, ck, row_tok, es);
    return hipGetLastError();
}

hipError_t launch_hisa_map(const sa_problem& p, int blk, int k_blocks, const int32_t* bidx, const int32_t* row_blk,
                           const int32_t* cidx, int32_t* idx, hipStream_t s) {
    const long n = (long)p.B * p.n_q * p.k;
    hipLaunchKernelGGL(hisa_map, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, blk, k_blocks, bidx, row_blk, cidx,
                       idx);
    return hipGetLastError();
}

}  // namespace sa
