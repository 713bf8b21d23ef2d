// Host side of libsa.so: argument validation, workspace layout and kernel dispatch.
// Every argument error is detected here, before anything is enqueued.
#include <math.h>
#include <atomic>
#include <string.h>

#include "sa_internal.h"

namespace {

using namespace sa;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int esize(int dtype) {
    switch (dtype) {
    case SA_F32: return 4;
    case SA_BF16: return 2;
    case SA_FP8_E4M3: return 1;
    default: return 0;
    }
}

bool problem_ok(const sa_problem* p) {
    if (!p) return false;
    if (p->B < 1 || p->n_q < 1 || p->n_kv < 1 || p->k < 1) return false;
    if (p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0) return false;
    if (p->d_qk < 1 || p->d_v < 1 || p->Hidx < 1 || p->d_idx < 1) return false;
    if (p->causal != 0 && p->causal != 1) return false;
    if (!(p->scale >= 0.f) || isinf(p->scale)) return false;
    // flat row counts must stay addressable with 32-bit grid dimensions
    if ((long long)p->B * p->n_q > 0x7fffffffLL) return false;
    return true;
}

// A strided view used with 16-byte vector loads of its contiguous last dimension.
sa_status tensor_ok(const sa_tensor& t, int last_dim, int ndims_strided) {
    const int es = esize(t.dtype);
    if (!t.data) return SA_ERR_INVALID_ARG;
    if (es == 0) return SA_ERR_UNSUPPORTED;
    if (((uintptr_t)t.data & 15) != 0) return SA_ERR_INVALID_ARG;
    const int64_t st[3] = {t.s0, t.s1, t.s2};
    for (int d = 0; d < ndims_strided; ++d) {
        if (st[d] < 0) return SA_ERR_INVALID_ARG;
        if ((st[d] * es) % 16 != 0) return SA_ERR_INVALID_ARG;
    }
    if (((int64_t)last_dim * es) % 16 != 0) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

sa_status ws_ok(const void* ws, size_t have, size_t need) {
    if (!ws) return SA_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255) != 0) return SA_ERR_WORKSPACE;
    if (have < need) return SA_ERR_WORKSPACE;
    return SA_OK;
}

size_t scores_bytes(const sa_problem& p) { return align256((size_t)p.B * p.n_q * p.n_kv * sizeof(float)); }
size_t idx_bytes(const sa_problem& p) { return align256((size_t)p.B * p.n_q * p.k * sizeof(int32_t)); }

sa_status check_indexer(const sa_problem* p, const sa_tensor& q, const sa_tensor& k, const sa_tensor& w) {
    sa_status s;
    if (q.dtype != SA_F32 && q.dtype != SA_BF16) return q.data ? SA_ERR_UNSUPPORTED : SA_ERR_INVALID_ARG;
    if (k.dtype != SA_F32 && k.dtype != SA_BF16 && k.dtype != SA_FP8_E4M3) return k.data ? SA_ERR_UNSUPPORTED : SA_ERR_INVALID_ARG;
    if (w.dtype != SA_F32) return w.data ? SA_ERR_UNSUPPORTED : SA_ERR_INVALID_ARG;
    if ((s = tensor_ok(q, p->d_idx, 3)) != SA_OK) return s;
    if ((s = tensor_ok(k, p->d_idx, 2)) != SA_OK) return s;
    if (!w.data || ((uintptr_t)w.data & 3)) return SA_ERR_INVALID_ARG;
    if (w.s0 < 0 || w.s1 < 0) return SA_ERR_INVALID_ARG;
    if ((long long)p->Hidx * p->d_idx > 8192) return SA_ERR_UNSUPPORTED;  // LDS staging of the plain path
    return SA_OK;
}

sa_status check_attn(const sa_problem* p, const sa_tensor& Q, const sa_tensor& K, const sa_tensor& V,
                     const sa_tensor& O) {
    sa_status s;
    if (Q.dtype != K.dtype || Q.dtype != V.dtype || Q.dtype != O.dtype) return SA_ERR_UNSUPPORTED;
    if (Q.dtype != SA_F32 && Q.dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if ((s = tensor_ok(Q, p->d_qk, 3)) != SA_OK) return s;
    if ((s = tensor_ok(K, p->d_qk, 3)) != SA_OK) return s;
    if ((s = tensor_ok(V, p->d_v, 3)) != SA_OK) return s;
    if ((s = tensor_ok(O, p->d_v, 3)) != SA_OK) return s;
    const int G = p->Hq / p->Hkv;
    if (attn_uses_mla(*p, Q.dtype)) return SA_OK;
    const int lpr = p->d_qk * esize(Q.dtype) / 16;
    if (p->d_qk != p->d_v) return SA_ERR_UNSUPPORTED;
    if (lpr != 8 && lpr != 16 && lpr != 32) return SA_ERR_UNSUPPORTED;
    if (G != 1 && G != 2 && G != 4) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

// Workspace of the hierarchical selection: status word, per-row block and candidate counts,
// block scores, kept-block lists, compact candidate keys, candidate scores and slots, top-k
// scratch.  R = B n_q rows, nb = n_kv / blk blocks, nc = (k_blocks + 1) blk candidates.
struct HisaLayout {
    size_t row_blk, row_tok, bscores, bidx, ckeys, cscores, cidx, scratch, total;
};
bool hisa_args_ok(const sa_problem* p, int blk, int k_blocks) {
    if (!problem_ok(p)) return false;
    if (blk != 16 && blk != 32 && blk != 64 && blk != 128 && blk != 256) return false;
    if (k_blocks < 1 || (long long)(k_blocks + 1) * blk > 32768) return false;
    return p->n_kv / blk >= 1;
}
sa_problem hisa_block_problem(const sa_problem& p, int blk, int k_blocks) {
    sa_problem q = p;
    q.n_kv = p.n_kv / blk;
    q.k = k_blocks;
    return q;
}
sa_problem hisa_token_problem(const sa_problem& p, int blk, int k_blocks) {
    sa_problem q = p;
    q.B = p.B * p.n_q;  // every row is its own batch over its own compact candidates
    q.n_q = 1;
    q.n_kv = (k_blocks + 1) * blk;
    q.causal = 0;
    q.kv_len = nullptr;
    q.q_pos0 = nullptr;
    return q;
}
HisaLayout hisa_layout(const sa_problem& p, int blk, int k_blocks, int k_es) {
    const size_t R = (size_t)p.B * p.n_q, nb = (size_t)(p.n_kv / blk), nc = (size_t)(k_blocks + 1) * blk;
    HisaLayout l;
    size_t o = kStatusBytes;
    l.row_blk = o; o += align256(R * 4);
    l.row_tok = o; o += align256(R * 4);
    l.bscores = o; o += align256(R * nb * 4);
    l.bidx = o; o += align256(R * (size_t)k_blocks * 4);
    l.ckeys = o; o += align256(R * nc * (size_t)p.d_idx * (size_t)k_es);
    l.cscores = o; o += align256(R * nc * 4);
    l.cidx = o; o += align256(R * (size_t)p.k * 4);
    const size_t t1 = topk_ws_bytes(hisa_block_problem(p, blk, k_blocks));
    const size_t t2 = topk_ws_bytes(hisa_token_problem(p, blk, k_blocks));
    l.scratch = o; o += align256(t1 > t2 ? t1 : t2);
    l.total = o;
    return l;
}

bool misa_args_ok(const sa_problem* p, int blk, int g) {
    if (!problem_ok(p)) return false;
    if (blk != 16 && blk != 32 && blk != 64 && blk != 128 && blk != 256) return false;
    if (g < 1 || g > p->Hidx || p->n_kv / blk < 1) return false;
    return misa_route_supported(*p);
}
sa_problem misa_head_problem(const sa_problem& p, int g) {
    sa_problem q = p;
    q.B = p.B * p.n_q;  // one selection of g heads out of Hidx per query row
    q.n_q = 1;
    q.n_kv = p.Hidx;
    q.k = g;
    q.causal = 0;
    q.kv_len = nullptr;
    q.q_pos0 = nullptr;
    return q;
}
// Workspace region of a selection (after the status word): the fused score + select's
// candidate lists, or the score rows and the top-k scratch.  A shape that the fused path
// takes but whose index dtypes it does not (f32 index queries or keys) scores and selects
// slices of at least 64 rows through the same region.
size_t select_slice_rows(const sa_problem& p, size_t region) { return region / ((size_t)p.n_kv * sizeof(float)); }
size_t select_region_bytes(const sa_problem& p) {
    if (select_fused_shape_ok(p)) {
        const size_t fused = select_fused_bytes(p), slice = (size_t)64 * p.n_kv * sizeof(float);
        return align256(fused > slice ? fused : slice);
    }
    return scores_bytes(p) + align256(topk_ws_bytes(p));
}

sa_status run_select(const sa_problem* p, const sa_tensor& q, const sa_tensor& k, const sa_tensor& w, int32_t* idx,
                     Status* status, char* region, hipStream_t st) {
    IndexerArgs ia;
    ia.p = *p;
    ia.q = q; ia.k = k; ia.w = w;
    ia.status = status;
    if (select_fused_ok(*p, q.dtype, k.dtype) && !env_flag("SA_FORCE_UNFUSED"))
        return launch_select_fused(ia, idx, region, st) == hipSuccess ? SA_OK : SA_ERR_HIP;
    TopkArgs ta;
    ta.p = *p;
    ta.idx = idx;
    ta.vals = nullptr;
    ta.status = status;
    ta.row_stride = p->n_kv;
    ia.row_stride = p->n_kv;
    ia.fill_invisible = 0;  // the selection reads only the visible prefix of each row
    ia.scores = reinterpret_cast<float*>(region);
    ta.scores = ia.scores;
    if (select_fused_shape_ok(*p)) {
        const long rows = (long)p->B * p->n_q;
        const long per = (long)select_slice_rows(*p, select_region_bytes(*p));
        for (long r0 = 0; r0 < rows; r0 += per) {
            ia.row0 = ta.row0 = (int)r0;
            ia.nrows = ta.nrows = (int)(rows - r0 < per ? rows - r0 : per);
            if (launch_indexer(ia, st) != hipSuccess) return SA_ERR_HIP;
            if (launch_topk(ta, st) != hipSuccess) return SA_ERR_HIP;
        }
        return SA_OK;
    }
    ta.scratch = region + scores_bytes(*p);
    if (topk_sliced(*p) && indexer_dec_path(ia)) {
        // few long rows: the index scan also fills the first radix digit of the selection
        if (topk_sliced_clear(ta, st) != hipSuccess) return SA_ERR_HIP;
        ia.hist0 = topk_sliced_hist(ta);
        ta.digit0_done = 1;
    }
    if (launch_indexer(ia, st) != hipSuccess) return SA_ERR_HIP;
    return launch_topk(ta, st) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// Workspace of the active-head selections (plain and with the shared linear term): status
// word, complete visible blocks per row, routing scores, active heads, the scored heads'
// queries and weights (Hs heads per row: misa_heads(g) for the active heads padded with zero
// heads, resmisa_heads(g) for the residual-head problem), top-k scratch of the head choice,
// the token selection's region.
struct MisaLayout {
    size_t row_blk, route, heads, qa, wa, scratch, region, total;
};
sa_problem scored_problem(const sa_problem& p, int Hs) {
    sa_problem q = p;
    q.Hidx = Hs;
    return q;
}
MisaLayout misa_layout(const sa_problem& p, int g, int Hs) {
    const size_t R = (size_t)p.B * p.n_q;
    MisaLayout l;
    size_t o = kStatusBytes;
    l.row_blk = o; o += align256(R * 4);
    l.route = o; o += align256(R * (size_t)p.Hidx * 4);
    l.heads = o; o += align256(R * (size_t)g * 4);
    l.qa = o; o += align256(R * (size_t)Hs * p.d_idx * 2);
    l.wa = o; o += align256(R * (size_t)Hs * 4);
    l.scratch = o; o += align256(topk_ws_bytes(misa_head_problem(p, g)));
    l.region = o; o += select_region_bytes(scored_problem(p, Hs));
    l.total = o;
    return l;
}

// Routing, head choice and the gather of the scored heads (plain active heads, or the
// residual-head problem), then the token selection over them.
sa_status misa_run(const sa_problem* p, const sa_tensor& q_idx, const sa_tensor& k_idx, const sa_tensor& w,
                   const uint16_t* kbar, int blk, int g, bool residual, int32_t* idx, int32_t* heads, char* base,
                   hipStream_t st) {
    const int Hs = residual ? resmisa_heads(g) : misa_heads(g);
    const MisaLayout l = misa_layout(*p, g, Hs);
    int32_t* row_blk = reinterpret_cast<int32_t*>(base + l.row_blk);
    float* route = reinterpret_cast<float*>(base + l.route);
    int32_t* hsel = heads ? heads : reinterpret_cast<int32_t*>(base + l.heads);
    uint16_t* qa = reinterpret_cast<uint16_t*>(base + l.qa);
    float* wa = reinterpret_cast<float*>(base + l.wa);
    Status* status = reinterpret_cast<Status*>(base);
    if (launch_hisa_rows(*p, blk, row_blk, st) != hipSuccess) return SA_ERR_HIP;
    if (launch_misa_route(*p, q_idx, w, kbar, blk, row_blk, route, st) != hipSuccess) return SA_ERR_HIP;
    TopkArgs th;  // g heads of Hidx per row, ranked by (routing score desc, head asc)
    th.p = misa_head_problem(*p, g);
    th.scores = route;
    th.row_stride = p->Hidx;
    th.idx = hsel;
    th.vals = nullptr;
    th.status = status;
    th.scratch = base + l.scratch;
    if (launch_topk(th, st) != hipSuccess) return SA_ERR_HIP;
    const hipError_t e = residual ? launch_resmisa_gather(*p, q_idx, w, g, hsel, qa, wa, st)
                                  : launch_misa_gather(*p, q_idx, w, g, hsel, qa, wa, st);
    if (e != hipSuccess) return SA_ERR_HIP;
    const sa_problem pa = scored_problem(*p, Hs);
    const sa_tensor qt{qa, SA_BF16, (int64_t)p->n_q * Hs * p->d_idx, (int64_t)Hs * p->d_idx, p->d_idx};
    const sa_tensor wt{wa, SA_F32, (int64_t)p->n_q * Hs, Hs, 0};
    return run_select(&pa, qt, k_idx, wt, idx, status, base + l.region, st);
}

float eff_scale(const sa_problem* p) { return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->d_qk); }

// Scratch of the entry point that allocates nothing (sa_select_attend_noalloc): a fixed
// array in device memory, one per GPU the library runs on, held until the process ends.
// Its device address comes from hipGetSymbolAddress once per device (the array's name is
// only a host-side stand-in); every call on a device shares that device's copy.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];

char* noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    char* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev].store(static_cast<char*>(ptr), std::memory_order_release);  // same value from any thread
    return static_cast<char*>(ptr);
}

// Block-table view of paged K/V pools (table null: K and V hold each batch's rows).
struct Pages {
    const int32_t* table = nullptr;
    int64_t stride = 0, pool_rows = 0;
    int shift = 0;
};

AttnArgs attn_args(const sa_problem* p, const sa_tensor& Q, const sa_tensor& K, const sa_tensor& V, const int32_t* idx,
                   const sa_tensor& O, float* lse, void* partial, const Pages& pg) {
    AttnArgs a;
    a.p = *p;
    a.Q = Q; a.K = K; a.V = V; a.O = O;
    a.idx = idx;
    a.lse = lse;
    a.scale = eff_scale(p);
    a.splits = attn_uses_mla(*p, Q.dtype) ? attn_splits(*p) : 1;
    a.partial = partial;
    a.lse_bs = (int64_t)p->Hq * p->n_q;
    a.block_table = pg.table;
    a.bt_stride = pg.stride;
    a.page_shift = pg.shift;
    a.pool_rows = pg.pool_rows;
    return a;
}

sa_status run_attn(const sa_problem* p, const sa_tensor& Q, const sa_tensor& K, const sa_tensor& V,
                   const int32_t* idx, const sa_tensor& O, float* lse, void* partial, hipStream_t st,
                   const Pages& pg = Pages(), int64_t lse_bs = 0) {
    AttnArgs a = attn_args(p, Q, K, V, idx, O, lse, partial, pg);
    if (lse_bs) a.lse_bs = lse_bs;
    return launch_attn(a, st) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// Grouped candidate sets: the problem of one group (Hq / G query heads, Hidx / G index heads,
// Hkv / G key/value heads, or the one shared key/value head).  Index-head groups start on
// 16-byte boundaries of w (Hidx / G a multiple of 4).
bool group_problem(const sa_problem* p, int G, sa_problem* out) {
    if (!problem_ok(p) || G < 1 || p->Hq % G != 0 || p->Hidx % G != 0) return false;
    sa_problem q = *p;
    q.Hq = p->Hq / G;
    q.Hidx = p->Hidx / G;
    if (G > 1 && q.Hidx % 4 != 0) return false;
    if (p->Hkv % G == 0) q.Hkv = p->Hkv / G;
    else if (p->Hkv == 1) q.Hkv = 1;
    else return false;
    *out = q;
    return true;
}
// Workspace of the grouped call: status word, the groups' selections (when the caller does
// not take them), the split partials, and one group's selection region (streaming lists or
// score rows, as for sa_select), reused group after group.
struct GroupedLayout {
    size_t idx, partial, region, total;
};
GroupedLayout grouped_layout(const sa_problem& p, const sa_problem& pg, int G) {
    GroupedLayout l;
    size_t o = kStatusBytes;
    l.idx = o; o += align256((size_t)G * p.B * p.n_q * p.k * sizeof(int32_t));
    l.partial = o; o += align256(attn_partial_bytes(pg));
    l.region = o; o += select_region_bytes(pg);
    l.total = o;
    return l;
}
char* offset_bytes(const void* base, int64_t bytes) { return const_cast<char*>(static_cast<const char*>(base)) + bytes; }

// Score, select and attend with the space after the status word at `body`: the selection
// (when the caller does not take it), the split partials, then the selection region.
sa_status select_attend_in(const sa_problem* p, const sa_tensor& q_idx, const sa_tensor& k_idx, const sa_tensor& w,
                           const sa_tensor& Q, const sa_tensor& K, const sa_tensor& V, int32_t* idx_out,
                           const sa_tensor& O, float* lse, Status* status, char* body, hipStream_t st) {
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(body);
    void* partial = body + idx_bytes(*p);
    char* region = static_cast<char*>(partial) + align256(attn_partial_bytes(*p));
    sa_status s = run_select(p, q_idx, k_idx, w, idx, status, region, st);
    if (s != SA_OK) return s;
    if (env_flag("SA_DEBUG_CHECKS") && launch_check_indices(*p, idx, status, st) != hipSuccess) return SA_ERR_HIP;
    return run_attn(p, Q, K, V, idx, O, lse, partial, st);
}

}  // namespace

extern "C" {

int sa_abi_version(void) { return SA_ABI_VERSION; }

const char* sa_status_str(sa_status s) {
    switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    case SA_ERR_NONFINITE: return "SA_ERR_NONFINITE";
    case SA_ERR_INDEX: return "SA_ERR_INDEX";
    default: return "SA_ERR_UNKNOWN";
    }
}

size_t sa_workspace_bytes(const sa_problem* p, int op) {
    if (!problem_ok(p)) return 0;
    switch (op) {
    case SA_OP_INDEXER_SCORE: return 0;
    case SA_OP_TOPK: return kStatusBytes + align256(topk_ws_bytes(*p));
    case SA_OP_SPARSE_ATTN: return kStatusBytes + align256(attn_partial_bytes(*p));
    case SA_OP_SPARSE_ATTN_PAGED: {
        // the latent kernel's split partials, or the multi-head kernel's translated rows
        const size_t part = align256(attn_partial_bytes(*p)), rows = idx_bytes(*p);
        return kStatusBytes + (part > rows ? part : rows);
    }
    case SA_OP_SELECT: return kStatusBytes + select_region_bytes(*p);
    case SA_OP_SELECT_ATTEND:
        return kStatusBytes + idx_bytes(*p) + align256(attn_partial_bytes(*p)) + select_region_bytes(*p);
    default: return 0;
    }
}

sa_status sa_indexer_score(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, float* scores,
                           void* stream) {
    if (!problem_ok(p) || !scores || ((uintptr_t)scores & 3)) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    IndexerArgs a;
    a.p = *p;
    a.q = q_idx; a.k = k_idx; a.w = w;
    a.scores = scores;
    a.row_stride = p->n_kv;
    a.fill_invisible = 1;
    a.status = nullptr;
    return launch_indexer(a, (hipStream_t)stream) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

sa_status sa_topk(const sa_problem* p, const float* scores, int64_t row_stride, int32_t* idx, float* vals, void* ws,
                  size_t ws_bytes, void* stream) {
    if (!problem_ok(p) || !scores || !idx || ((uintptr_t)scores & 3)) return SA_ERR_INVALID_ARG;
    if (row_stride < p->n_kv) return SA_ERR_INVALID_ARG;
    sa_status s = ws_ok(ws, ws_bytes, sa_workspace_bytes(p, SA_OP_TOPK));
    if (s != SA_OK) return s;
    TopkArgs a;
    a.p = *p;
    a.scores = scores;
    a.row_stride = row_stride;
    a.idx = idx;
    a.vals = vals;
    a.status = static_cast<Status*>(ws);
    a.scratch = static_cast<char*>(ws) + kStatusBytes;
    return launch_topk(a, (hipStream_t)stream) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

sa_status sa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, int32_t* idx, void* ws,
                    size_t ws_bytes, void* stream) {
    if (!problem_ok(p) || !idx || ((uintptr_t)idx & 3)) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    if ((s = ws_ok(ws, ws_bytes, sa_workspace_bytes(p, SA_OP_SELECT))) != SA_OK) return s;
    char* base = static_cast<char*>(ws);
    return run_select(p, q_idx, k_idx, w, idx, reinterpret_cast<Status*>(base), base + kStatusBytes,
                      (hipStream_t)stream);
}

sa_status sa_sparse_attn(const sa_problem* p, sa_tensor Q, sa_tensor K, sa_tensor V, const int32_t* idx, sa_tensor O,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (!problem_ok(p) || !idx || ((uintptr_t)idx & 3)) return SA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3)) return SA_ERR_INVALID_ARG;
    sa_status s = check_attn(p, Q, K, V, O);
    if (s != SA_OK) return s;
    if ((s = ws_ok(ws, ws_bytes, sa_workspace_bytes(p, SA_OP_SPARSE_ATTN))) != SA_OK) return s;
    void* partial = static_cast<char*>(ws) + kStatusBytes;
    if (env_flag("SA_DEBUG_CHECKS") &&
        launch_check_indices(*p, idx, reinterpret_cast<Status*>(ws), (hipStream_t)stream) != hipSuccess)
        return SA_ERR_HIP;
    return run_attn(p, Q, K, V, idx, O, lse, partial, (hipStream_t)stream);
}

sa_status sa_sparse_attn_paged(const sa_problem* p, sa_tensor Q, sa_tensor K, sa_tensor V, int64_t pool_rows,
                               const int32_t* block_table, int64_t bt_stride, int page_size, const int32_t* idx,
                               sa_tensor O, float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (!problem_ok(p) || !idx || ((uintptr_t)idx & 3)) return SA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3)) return SA_ERR_INVALID_ARG;
    if (!block_table || ((uintptr_t)block_table & 3)) return SA_ERR_INVALID_ARG;
    if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0) return SA_ERR_INVALID_ARG;
    if (pool_rows < 1 || bt_stride < ((int64_t)p->n_kv + page_size - 1) / page_size) return SA_ERR_INVALID_ARG;
    sa_status s = check_attn(p, Q, K, V, O);
    if (s != SA_OK) return s;
    if ((s = ws_ok(ws, ws_bytes, sa_workspace_bytes(p, SA_OP_SPARSE_ATTN_PAGED))) != SA_OK) return s;
    Pages pg;
    pg.table = block_table;
    pg.stride = bt_stride;
    pg.pool_rows = pool_rows;
    while ((1 << pg.shift) < page_size) ++pg.shift;
    void* partial = static_cast<char*>(ws) + kStatusBytes;
    if (!attn_paged_ok(attn_args(p, Q, K, V, idx, O, lse, partial, pg))) return SA_ERR_UNSUPPORTED;
    if (env_flag("SA_DEBUG_CHECKS") &&
        launch_check_indices(*p, idx, reinterpret_cast<Status*>(ws), (hipStream_t)stream) != hipSuccess)
        return SA_ERR_HIP;
    return run_attn(p, Q, K, V, idx, O, lse, partial, (hipStream_t)stream, pg);
}

sa_status sa_select_attend(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, sa_tensor Q,
                           sa_tensor K, sa_tensor V, int32_t* idx_out, sa_tensor O, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
    if (!problem_ok(p)) return SA_ERR_INVALID_ARG;
    if (idx_out && ((uintptr_t)idx_out & 3)) return SA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3)) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    if ((s = check_attn(p, Q, K, V, O)) != SA_OK) return s;
    if ((s = ws_ok(ws, ws_bytes, sa_workspace_bytes(p, SA_OP_SELECT_ATTEND))) != SA_OK) return s;
    char* base = static_cast<char*>(ws);
    return select_attend_in(p, q_idx, k_idx, w, Q, K, V, idx_out, O, lse, reinterpret_cast<Status*>(base),
                            base + kStatusBytes, (hipStream_t)stream);
}

sa_status sa_select_attend_noalloc(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, sa_tensor Q,
                                   sa_tensor K, sa_tensor V, int32_t* idx_out, sa_tensor O, float* lse,
                                   uint32_t* status, void* stream) {
    if (!problem_ok(p)) return SA_ERR_INVALID_ARG;
    if (idx_out && ((uintptr_t)idx_out & 3)) return SA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3)) return SA_ERR_INVALID_ARG;
    if (status && ((uintptr_t)status & 255)) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    if ((s = check_attn(p, Q, K, V, O)) != SA_OK) return s;
    if (sa_workspace_bytes(p, SA_OP_SELECT_ATTEND) > kNoAllocScratchBytes) return SA_ERR_WORKSPACE;
    char* base = noalloc_scratch();
    if (!base) return SA_ERR_HIP;
    // the caller's status word, or the scratch's own (then nothing reports non-finite inputs)
    Status* st_word = status ? reinterpret_cast<Status*>(status) : reinterpret_cast<Status*>(base);
    return select_attend_in(p, q_idx, k_idx, w, Q, K, V, idx_out, O, lse, st_word, base + kStatusBytes,
                            (hipStream_t)stream);
}

size_t sa_grouped_workspace_bytes(const sa_problem* p, int groups) {
    sa_problem pg;
    if (!group_problem(p, groups, &pg)) return 0;
    return grouped_layout(*p, pg, groups).total;
}

sa_status sa_select_attend_grouped(const sa_problem* p, int groups, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w,
                                   sa_tensor Q, sa_tensor K, sa_tensor V, int32_t* idx_out, sa_tensor O, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
    sa_problem pg;
    if (!group_problem(p, groups, &pg)) return SA_ERR_INVALID_ARG;
    if (idx_out && ((uintptr_t)idx_out & 15)) return SA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3)) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    if ((s = check_attn(&pg, Q, K, V, O)) != SA_OK) return s;
    if ((s = ws_ok(ws, ws_bytes, sa_grouped_workspace_bytes(p, groups))) != SA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    const GroupedLayout L = grouped_layout(*p, pg, groups);
    char* base = static_cast<char*>(ws);
    int32_t* idx_all = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + L.idx);
    const int64_t per_group = (int64_t)p->B * p->n_q * p->k;
    const int eq = esize(q_idx.dtype), em = esize(Q.dtype);
    for (int g = 0; g < groups; ++g) {
        // the group's index heads: a view starting g Hidx/G heads in (w's heads are contiguous)
        sa_tensor qg = q_idx, wg = w;
        qg.data = offset_bytes(q_idx.data, (int64_t)g * pg.Hidx * q_idx.s2 * eq);
        wg.data = offset_bytes(w.data, (int64_t)g * pg.Hidx * 4);
        int32_t* idx = idx_all + g * per_group;
        if ((s = run_select(&pg, qg, k_idx, wg, idx, reinterpret_cast<Status*>(base), base + L.region, st)) != SA_OK)
            return s;
        // the group's query heads, their key/value heads (or the one shared head), O and lse
        sa_tensor Qg = Q, Og = O, Kg = K, Vg = V;
        Qg.data = offset_bytes(Q.data, (int64_t)g * pg.Hq * Q.s1 * em);
        Og.data = offset_bytes(O.data, (int64_t)g * pg.Hq * O.s1 * em);
        if (p->Hkv > 1) {
            Kg.data = offset_bytes(K.data, (int64_t)g * pg.Hkv * K.s1 * em);
            Vg.data = offset_bytes(V.data, (int64_t)g * pg.Hkv * V.s1 * em);
        }
        float* lg = lse ? lse + (int64_t)g * pg.Hq * p->n_q : nullptr;
        if ((s = run_attn(&pg, Qg, Kg, Vg, idx, Og, lg, base + L.partial, st, Pages(), (int64_t)p->Hq * p->n_q)) != SA_OK)
            return s;
    }
    return SA_OK;
}

sa_status sa_block_means(const sa_problem* p, sa_tensor k_idx, int blk, uint16_t* kbar, void* stream) {
    if (!problem_ok(p) || !kbar || ((uintptr_t)kbar & 15)) return SA_ERR_INVALID_ARG;
    if (blk != 16 && blk != 32 && blk != 64 && blk != 128 && blk != 256) return SA_ERR_INVALID_ARG;
    if (k_idx.dtype != SA_F32 && k_idx.dtype != SA_BF16 && k_idx.dtype != SA_FP8_E4M3)
        return k_idx.data ? SA_ERR_UNSUPPORTED : SA_ERR_INVALID_ARG;
    sa_status s = tensor_ok(k_idx, p->d_idx, 2);
    if (s != SA_OK) return s;
    if (p->d_idx > 256) return SA_ERR_UNSUPPORTED;
    return launch_block_means(*p, k_idx, blk, kbar, (hipStream_t)stream) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

size_t sa_hisa_workspace_bytes(const sa_problem* p, int blk, int k_blocks) {
    if (!hisa_args_ok(p, blk, k_blocks)) return 0;
    return hisa_layout(*p, blk, k_blocks, 4).total;  // sized for the widest key dtype
}

sa_status sa_hisa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, const uint16_t* kbar,
                         int blk, int k_blocks, int32_t* idx, int32_t* blocks, void* ws, size_t ws_bytes,
                         void* stream) {
    if (!hisa_args_ok(p, blk, k_blocks)) return SA_ERR_INVALID_ARG;
    if (!kbar || ((uintptr_t)kbar & 15) || !idx || ((uintptr_t)idx & 3)) return SA_ERR_INVALID_ARG;
    if (blocks && ((uintptr_t)blocks & 3)) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    // rows of all batches equally spaced: each row can stand as its own batch
    if (q_idx.s0 != (int64_t)p->n_q * q_idx.s1 || w.s0 != (int64_t)p->n_q * w.s1) return SA_ERR_UNSUPPORTED;
    if ((s = ws_ok(ws, ws_bytes, sa_hisa_workspace_bytes(p, blk, k_blocks))) != SA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    const int es = esize(k_idx.dtype);
    const HisaLayout l = hisa_layout(*p, blk, k_blocks, es);
    int32_t* row_blk = reinterpret_cast<int32_t*>(base + l.row_blk);
    int32_t* row_tok = reinterpret_cast<int32_t*>(base + l.row_tok);
    float* bscores = reinterpret_cast<float*>(base + l.bscores);
    int32_t* bidx = blocks ? blocks : reinterpret_cast<int32_t*>(base + l.bidx);
    uint8_t* ckeys = reinterpret_cast<uint8_t*>(base + l.ckeys);
    float* cscores = reinterpret_cast<float*>(base + l.cscores);
    int32_t* cidx = reinterpret_cast<int32_t*>(base + l.cidx);
    Status* status = reinterpret_cast<Status*>(base);
    const sa_problem pb = hisa_block_problem(*p, blk, k_blocks);
    const sa_problem pt = hisa_token_problem(*p, blk, k_blocks);

    if (launch_hisa_rows(*p, blk, row_blk, st) != hipSuccess) return SA_ERR_HIP;
    // block scores over the representatives; visible blocks = complete blocks of the prefix
    IndexerArgs ia;
    ia.p = pb;
    ia.q = q_idx; ia.w = w;
    ia.k = sa_tensor{const_cast<uint16_t*>(kbar), SA_BF16, (int64_t)pb.n_kv * p->d_idx, p->d_idx, 0};
    ia.scores = bscores;
    ia.row_stride = pb.n_kv;
    ia.fill_invisible = 0;
    ia.status = nullptr;  // non-finite scores stay visible and are reported by the selection
    ia.row_len = row_blk;
    if (launch_indexer(ia, st) != hipSuccess) return SA_ERR_HIP;
    TopkArgs ta;
    ta.p = pb;
    ta.scores = bscores;
    ta.row_stride = pb.n_kv;
    ta.idx = bidx;
    ta.vals = nullptr;
    ta.status = status;
    ta.scratch = base + l.scratch;
    ta.row_len = row_blk;
    if (launch_topk(ta, st) != hipSuccess) return SA_ERR_HIP;
    // the kept blocks and the open block of every row as compact candidate keys
    if (launch_hisa_gather(*p, k_idx, blk, k_blocks, bidx, row_blk, ckeys, row_tok, st) != hipSuccess) return SA_ERR_HIP;
    IndexerArgs ib;
    ib.p = pt;
    ib.q = sa_tensor{q_idx.data, q_idx.dtype, q_idx.s1, q_idx.s1, q_idx.s2};
    ib.w = sa_tensor{w.data, w.dtype, w.s1, w.s1, 0};
    ib.k = sa_tensor{ckeys, k_idx.dtype, (int64_t)pt.n_kv * p->d_idx, p->d_idx, 0};
    ib.scores = cscores;
    ib.row_stride = pt.n_kv;
    ib.fill_invisible = 0;
    ib.status = nullptr;
    ib.row_len = row_tok;
    if (launch_indexer(ib, st) != hipSuccess) return SA_ERR_HIP;
    TopkArgs tb;
    tb.p = pt;
    tb.scores = cscores;
    tb.row_stride = pt.n_kv;
    tb.idx = cidx;
    tb.vals = nullptr;
    tb.status = status;
    tb.scratch = base + l.scratch;
    tb.row_len = row_tok;
    if (launch_topk(tb, st) != hipSuccess) return SA_ERR_HIP;
    return launch_hisa_map(*p, blk, k_blocks, bidx, row_blk, cidx, idx, st) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

size_t sa_misa_workspace_bytes(const sa_problem* p, int blk, int g) {
    if (!misa_args_ok(p, blk, g)) return 0;
    return misa_layout(*p, g, misa_heads(g)).total;
}

sa_status sa_misa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, const uint16_t* kbar,
                         int blk, int g, int32_t* idx, int32_t* heads, void* ws, size_t ws_bytes, void* stream) {
    if (!problem_ok(p) || !kbar || ((uintptr_t)kbar & 15) || !idx || ((uintptr_t)idx & 3)) return SA_ERR_INVALID_ARG;
    if (heads && ((uintptr_t)heads & 3)) return SA_ERR_INVALID_ARG;
    if (blk != 16 && blk != 32 && blk != 64 && blk != 128 && blk != 256) return SA_ERR_INVALID_ARG;
    if (g < 1 || g > p->Hidx || p->n_kv / blk < 1) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    if (q_idx.dtype != SA_BF16 || !misa_route_supported(*p)) return SA_ERR_UNSUPPORTED;
    if ((s = ws_ok(ws, ws_bytes, sa_misa_workspace_bytes(p, blk, g))) != SA_OK) return s;
    return misa_run(p, q_idx, k_idx, w, kbar, blk, g, false, idx, heads, static_cast<char*>(ws), (hipStream_t)stream);
}

size_t sa_resmisa_workspace_bytes(const sa_problem* p, int blk, int g) {
    if (!misa_args_ok(p, blk, g) || g + 6 > 64) return 0;
    return misa_layout(*p, g, resmisa_heads(g)).total;
}

sa_status sa_resmisa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, const uint16_t* kbar,
                            int blk, int g, int32_t* idx, int32_t* heads, void* ws, size_t ws_bytes, void* stream) {
    if (!problem_ok(p) || !kbar || ((uintptr_t)kbar & 15) || !idx || ((uintptr_t)idx & 3)) return SA_ERR_INVALID_ARG;
    if (heads && ((uintptr_t)heads & 3)) return SA_ERR_INVALID_ARG;
    if (blk != 16 && blk != 32 && blk != 64 && blk != 128 && blk != 256) return SA_ERR_INVALID_ARG;
    if (g < 1 || g > p->Hidx || g + 6 > 64 || p->n_kv / blk < 1) return SA_ERR_INVALID_ARG;
    sa_status s = check_indexer(p, q_idx, k_idx, w);
    if (s != SA_OK) return s;
    if (q_idx.dtype != SA_BF16 || !misa_route_supported(*p)) return SA_ERR_UNSUPPORTED;
    if ((s = ws_ok(ws, ws_bytes, sa_resmisa_workspace_bytes(p, blk, g))) != SA_OK) return s;
    return misa_run(p, q_idx, k_idx, w, kbar, blk, g, true, idx, heads, static_cast<char*>(ws), (hipStream_t)stream);
}

sa_status sa_device_status(void* ws, void* stream) {
    if (!ws || ((uintptr_t)ws & 255)) return SA_ERR_WORKSPACE;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SA_ERR_HIP;
    Status st;
    if (hipMemcpy(&st, ws, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return SA_ERR_HIP;
    Status zero;
    zero.flags = 0;
    if (hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return SA_ERR_HIP;
    if (st.flags & (1u << SA_ERR_NONFINITE)) return SA_ERR_NONFINITE;
    if (st.flags & (1u << SA_ERR_INDEX)) return SA_ERR_INDEX;
    return SA_OK;
}

}  // extern "C"
