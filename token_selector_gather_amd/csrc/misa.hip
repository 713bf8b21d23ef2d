// Active index heads: routing scores and the gather of each query's active heads.
//
// "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the MISA paragraphs: every query keeps g of its
// G index heads, chosen from the block-averaged index keys (the absolute value of each
// head's weighted ReLU response, averaged over the blocks of the current prefix), and the
// score then sums only those heads.  The head choice and the scores reuse the top-k and
// indexer kernels; the kernels here compute the routing scores and gather the chosen heads:
//  * misa_route: route[r][h] = |w_h| * mean over the complete visible blocks B of
//    ReLU(<q_h, kbar_B>), with kbar the bf16 block representatives of the hierarchical
//    selection; 0 for a row without a complete visible block.  One workgroup per query
//    row: the G x d_idx query in MFMA A fragments (rows = heads), 16 representatives per
//    B fragment read straight from memory (a batch's representatives stay in L2), the
//    ReLU'd products summed per head in registers, then across the 16 lanes of a head and
//    the four waves in a fixed order;
//  * misa_gather: the active heads' index queries and weights, in ascending head order,
//    then zero heads up to 16, 32 or 64.
//  * resmisa_gather (the ResMiSA paragraph of the same section: ReLU(z) = z + ReLU(-z) makes
//    the heads' linear terms ONE shared dot product, and only some heads keep their
//    non-linear residual): the query heads of a derived indexer problem whose score is
//    <qbar, k> + sum_{h active} w_h ReLU(-<q_h, k>) with qbar = sum_h w_h q_h:
//      slots 0 .. g-1    residual heads, query -q_h (exact bf16 negation), weight w_h;
//      slots g .. g+5    the shared term: qbar in fp32 split exactly into three bf16 parts
//                        b1 + b2 + b3, each as the pair (b, +1), (-b, -1), since
//                        ReLU(<b, k>) - ReLU(<-b, k>) = <b, k>;
//      the rest          zero query and weight (padding to the indexer's 16 / 32 / 64 heads).
//    qbar is summed in fp32 in ascending head order; the split is exact for normal values
//    (each part takes the next 8 significant bits), so the indexer's fp32 accumulation sees
//    the shared query to fp32 precision.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

template <int KSTEPS, int H>
__global__ void __launch_bounds__(256) misa_route(sa_problem p, sa_tensor q, sa_tensor w, const uint16_t* kbar, int nb,
                                                  const int32_t* row_blk, float* route) {
    constexpr int MT = H / 16;
    constexpr int D = 32 * KSTEPS;
    __shared__ float s_part[4][H];
    const int lane = threadIdx.x & 63, l15 = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long r = blockIdx.x;
    const int b = (int)(r / p.n_q), i = (int)(r % p.n_q);
    const int P = row_blk[r];
    float rs[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) rs[m][e] = 0.f;
    if (P > 0) {
        // A fragments: row 16 m + lane%16 = head, k-step s holds d = 32 s + 8 (lane/16) + 0..7
        bf16x8 av[MT][KSTEPS];
        const uint16_t* qp = static_cast<const uint16_t*>(q.data) + b * q.s0 + (int64_t)i * q.s1;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
                av[m][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + (16 * m + l15) * q.s2 + 32 * s + 8 * g));
        const uint16_t* kb = kbar + (int64_t)b * nb * D;
        const int ntl = (P + 15) / 16;
        for (int u = wv; u < ntl; u += 4) {
            const int blk_id = 16 * u + l15;  // this lane's column: representative blk_id
            const bool ok = blk_id < P;
            const uint16_t* kr = kb + (int64_t)(ok ? blk_id : 0) * D + 8 * g;
            f32x4 acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + 32 * s));
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][s], bv, acc[m], 0, 0, 0);
            }
            // acc[m][e]: head 16 m + 4 (lane/16) + e against representative blk_id
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) rs[m][e] += ok ? fmaxf(acc[m][e], 0.f) : 0.f;
        }
    }
    // sum over the 16 representatives of a lane row, then over the waves
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = rs[m][e];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
            if (l15 == 0) s_part[wv][16 * m + 4 * g + e] = v;
        }
    __syncthreads();
    if (threadIdx.x < H) {
        const int h = threadIdx.x;
        const float sum = ((s_part[0][h] + s_part[1][h]) + s_part[2][h]) + s_part[3][h];
        const float wh = fabsf(static_cast<const float*>(w.data)[b * w.s0 + (int64_t)i * w.s1 + h]);
        route[r * H + h] = P > 0 ? wh * (sum / (float)P) : 0.f;
    }
}

// thread (r, j, piece): piece of slot j of row r (16 bytes of a bf16 query); slots g .. Hs-1
// are zero heads
__global__ void __launch_bounds__(256) misa_gather(sa_problem p, sa_tensor q, sa_tensor w, int g, int Hs,
                                                   const int32_t* heads, uint16_t* qa, float* wa) {
    const int pieces = p.d_idx / 8;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)p.B * p.n_q * Hs * pieces) return;
    const int c = (int)(e % pieces);
    const long rj = e / pieces;
    const long r = rj / Hs;
    const int j = (int)(rj % Hs);
    const int b = (int)(r / p.n_q), i = (int)(r % p.n_q);
    uint4 v = make_uint4(0, 0, 0, 0);
    float wv = 0.f;
    if (j < g) {
        const int h = heads[r * g + j];
        v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q.data) + b * q.s0 + (int64_t)i * q.s1 +
                                            (int64_t)h * q.s2 + 8 * c);
        wv = static_cast<const float*>(w.data)[b * w.s0 + (int64_t)i * w.s1 + h];
    }
    *reinterpret_cast<uint4*>(qa + rj * p.d_idx + 8 * c) = v;
    if (c == 0) wa[rj] = wv;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// one workgroup of d_idx threads per query row; thread t owns element t of every slot
__global__ void __launch_bounds__(128) resmisa_gather(sa_problem p, sa_tensor q, sa_tensor w, int g, int Hp,
                                                      const int32_t* heads, uint16_t* qa, float* wa) {
    const long r = blockIdx.x;
    const int b = (int)(r / p.n_q), i = (int)(r % p.n_q);
    const int t = threadIdx.x;
    const uint16_t* qr = static_cast<const uint16_t*>(q.data) + b * q.s0 + (int64_t)i * q.s1;
    const float* wr = static_cast<const float*>(w.data) + b * w.s0 + (int64_t)i * w.s1;
    uint16_t* out = qa + r * (int64_t)Hp * p.d_idx;
    float qbar = 0.f;
    for (int h = 0; h < p.Hidx; ++h) qbar = fmaf(wr[h], bf16_val(qr[(int64_t)h * q.s2 + t]), qbar);
    const uint16_t b1 = bf16_rne(qbar);
    const float r1 = qbar - bf16_val(b1);
    const uint16_t b2 = bf16_rne(r1);
    const uint16_t b3 = bf16_rne(r1 - bf16_val(b2));
    const uint16_t part[3] = {b1, b2, b3};
    for (int j = 0; j < g; ++j) {
        const int h = heads[r * g + j];
        out[(int64_t)j * p.d_idx + t] = qr[(int64_t)h * q.s2 + t] ^ 0x8000u;
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        out[(int64_t)(g + 2 * m) * p.d_idx + t] = part[m];
        out[(int64_t)(g + 2 * m + 1) * p.d_idx + t] = part[m] ^ 0x8000u;
    }
    for (int j = g + 6; j < Hp; ++j) out[(int64_t)j * p.d_idx + t] = 0;
    float* wo = wa + r * Hp;
    if (t < g) wo[t] = wr[heads[r * g + t]];
    else if (t < g + 6) wo[t] = ((t - g) & 1) ? -1.f : 1.f;
    else if (t < Hp) wo[t] = 0.f;
}

}  // namespace

bool misa_route_supported(const sa_problem& p) {
    return (p.Hidx == 16 || p.Hidx == 32 || p.Hidx == 64) && (p.d_idx == 64 || p.d_idx == 128);
}

hipError_t launch_misa_route(const sa_problem& p, const sa_tensor& q, const sa_tensor& w, const uint16_t* kbar, int blk,
                             const int32_t* row_blk, float* route, hipStream_t s) {
    const int nb = p.n_kv / blk;
    const dim3 grid((unsigned)((long)p.B * p.n_q)), block(256);
#define SA_ROUTE(KS, HH)                                                                         \
    if (p.Hidx == HH) {                                                                          \
        hipLaunchKernelGGL((misa_route<KS, HH>), grid, block, 0, s, p, q, w, kbar, nb, row_blk, route); \
        return hipGetLastError();                                                                \
    }
    if (p.d_idx == 64) { SA_ROUTE(2, 16) SA_ROUTE(2, 32) SA_ROUTE(2, 64) }
    else { SA_ROUTE(4, 16) SA_ROUTE(4, 32) SA_ROUTE(4, 64) }
#undef SA_ROUTE
    return hipErrorInvalidValue;
}

hipError_t launch_misa_gather(const sa_problem& p, const sa_tensor& q, const sa_tensor& w, int g, const int32_t* heads,
                              uint16_t* qa, float* wa, hipStream_t s) {
    const int Hs = misa_heads(g);
    const long n = (long)p.B * p.n_q * Hs * (p.d_idx / 8);
    hipLaunchKernelGGL(misa_gather, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, q, w, g, Hs, heads, qa, wa);
    return hipGetLastError();
}

}  // namespace sa

namespace sa {
int misa_heads(int g) { return g <= 16 ? 16 : (g <= 32 ? 32 : 64); }
int resmisa_heads(int g) { return misa_heads(g + 6); }

hipError_t launch_resmisa_gather(const sa_problem& p, const sa_tensor& q, const sa_tensor& w, int g, const int32_t* heads,
                                 uint16_t* qa, float* wa, hipStream_t s) {
    const int Hp = resmisa_heads(g);
    hipLaunchKernelGGL(resmisa_gather, dim3((unsigned)((long)p.B * p.n_q)), dim3(p.d_idx), 0, s, p, q, w, g, Hp, heads,
                       qa, wa);
    return hipGetLastError();
}
}  // namespace sa
