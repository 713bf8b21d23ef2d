// Internal declarations shared by the host dispatcher and the kernels of libsa.so.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <stdint.h>

#include "sa.h"

namespace sa {

// Visible-history description of one batch, read on the device from kv_len / q_pos0.
struct Rows {
    const int32_t* kv_len;  // [B] or null (= n_kv)
    const int32_t* q_pos0;  // [B] or null (= 0)
    int32_t n_q, n_kv, causal;
    const int32_t* row_len = nullptr;  // [B * n_q] or null: explicit visible lengths (derived
                                       // problems of the hierarchical selection)
};

// Number of visible history positions of query row (b, i); 0 for an invalid row.  The
// visible set is always the prefix [0, L) of the history.
__device__ __forceinline__ int visible_len(const Rows& r, int b, int i) {
    if (r.row_len) return r.row_len[(long)b * r.n_q + i];
    int kl = r.kv_len ? r.kv_len[b] : r.n_kv;
    kl = kl < 0 ? 0 : (kl > r.n_kv ? r.n_kv : kl);
    long qp = (long)(r.q_pos0 ? r.q_pos0[b] : 0) + i;
    if (qp < 0 || qp >= kl) return 0;
    if (!r.causal) return kl;
    long L = qp + 1;
    return (int)(L < kl ? L : kl);
}

// Status word layout at the start of every workspace.
constexpr size_t kStatusBytes = 256;
struct Status {
    uint32_t flags;  // bit SA_ERR_NONFINITE set when a visible score was not finite
};

// --- launchers (each returns hipSuccess or the launch error) ---

struct IndexerArgs {
    sa_problem p;
    sa_tensor q, k, w;
    float* scores;
    int64_t row_stride;  // floats between consecutive rows of scores
    int fill_invisible;  // 1: write -inf into every invisible entry of [0, n_kv)
    Status* status;      // fused call: non-finite index inputs are reported here by a pre-pass,
                         // and the score kernel may clip NaN with a plain max; null: the visible
                         // scores of rows and keys with non-finite inputs come out non-finite
    int fix_nonfinite = 0;  // set by the launcher: the plain-max kernel writes NaN for query rows
                            // with non-finite inputs, and a later pass for such keys
    const int32_t* row_len = nullptr;  // explicit visible length per row (see Rows)
    int row0 = 0, nrows = 0;  // nrows > 0: only flat rows [row0, row0 + nrows), whose scores start at
                              // `scores` (the plain vector path only)
    uint32_t* hist0 = nullptr;  // (few-row layout only, see indexer_dec_path) the sliced top-k's
                                // per-row histograms: the scan adds the first digit of every
                                // visible score and reports non-finite scores in `status`
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s);
// The indexer takes its few-row layout (indexer_dec), the one that can fill hist0.
bool indexer_dec_path(const IndexerArgs& a);

// Fused score + select for many query rows (the prefill layout of the indexer with a
// streaming top-k instead of stored scores).  A persistent grid of at most kSelSlots
// workgroups; workgroup w keeps the candidate lists of its rows in slice w of `buf`.
constexpr int kSelSlots = 512;
struct SelectArgs {
    uint32_t* buf = nullptr;  // select_fused_bytes(p) bytes
    int cap = 0;              // candidate entries per row
    int32_t* idx = nullptr;   // [B, n_q, k] output
};
bool select_fused_ok(const sa_problem& p, int q_dtype, int k_dtype);  // dtypes and shape
bool select_fused_shape_ok(const sa_problem& p);                       // shape only
size_t select_fused_bytes(const sa_problem& p);
// a.status must be set: non-finite index inputs are reported there
hipError_t launch_select_fused(const IndexerArgs& a, int32_t* idx, void* buf, hipStream_t s);

struct TopkArgs {
    sa_problem p;
    const float* scores;
    int64_t row_stride;
    int32_t* idx;
    float* vals;
    Status* status;
    void* scratch;  // topk_ws_bytes(p) bytes of workspace (per-row histograms of the sliced path)
    const int32_t* row_len = nullptr;  // explicit visible length per row (see Rows)
    int row0 = 0, nrows = 0;  // nrows > 0: only flat rows [row0, row0 + nrows), whose scores start at
                              // `scores` (the one-workgroup-per-row kernels only)
    int digit0_done = 0;  // sliced path: the histograms were cleared (topk_sliced_clear) before the
                          // scores were written and hold the first digit already (indexer hist0)
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
size_t topk_ws_bytes(const sa_problem& p);
bool topk_sliced(const sa_problem& p);
// The sliced path's per-row histograms in its scratch, and a kernel that clears them.
uint32_t* topk_sliced_hist(const TopkArgs& a);
hipError_t topk_sliced_clear(const TopkArgs& a, hipStream_t s);

struct AttnArgs {
    sa_problem p;
    sa_tensor Q, K, V, O;
    const int32_t* idx;
    float* lse;
    float scale;
    void* partial;  // workspace for split-candidate partial results (may be null if splits == 1)
    int splits;
    // paged K/V: logical position j of batch b lives in physical row
    // block_table[b * bt_stride + (j >> page_shift)] << page_shift | j % page size of page
    // pools indexed (head, physical row) without a batch offset; null: contiguous per batch
    const int32_t* block_table = nullptr;
    int64_t bt_stride = 0;
    int page_shift = 0;
    int64_t pool_rows = 0;
    int64_t lse_bs = 0;  // floats between batches of lse (Hq n_q for a whole call; more when
                         // the call covers one group of a tensor's heads)
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);

// Hierarchical selection (block representatives, then tokens inside the kept blocks).
hipError_t launch_block_means(const sa_problem& p, const sa_tensor& k, int blk, uint16_t* kbar, hipStream_t s);
// row_blk[r] = complete visible blocks of row r
hipError_t launch_hisa_rows(const sa_problem& p, int blk, int32_t* row_blk, hipStream_t s);
// compact candidate keys of every row (kept blocks in ascending order, then the open block),
// their count in row_tok
hipError_t launch_hisa_gather(const sa_problem& p, const sa_tensor& k, int blk, int k_blocks, const int32_t* bidx,
                              const int32_t* row_blk, uint8_t* ck, int32_t* row_tok, hipStream_t s);
// candidate slots -> history positions
hipError_t launch_hisa_map(const sa_problem& p, int blk, int k_blocks, const int32_t* bidx, const int32_t* row_blk,
                           const int32_t* cidx, int32_t* idx, hipStream_t s);

// Active index heads: routing scores over the block representatives, and the gather of the
// chosen heads' queries and weights.
bool misa_route_supported(const sa_problem& p);
hipError_t launch_misa_route(const sa_problem& p, const sa_tensor& q, const sa_tensor& w, const uint16_t* kbar, int blk,
                             const int32_t* row_blk, float* route, hipStream_t s);
// Scored heads of the derived indexer problem: the g active heads padded with zero heads to
// misa_heads(g) (16, 32 or 64, the head counts the streaming selection takes; a zero head
// adds exactly +0 to every score).
int misa_heads(int g);
hipError_t launch_misa_gather(const sa_problem& p, const sa_tensor& q, const sa_tensor& w, int g, const int32_t* heads,
                              uint16_t* qa, float* wa, hipStream_t s);
// Shared linear term + residual heads: the derived problem's heads (resmisa_heads(g) of them:
// g residual heads, six parts of the shared query, zero padding), queries and weights.
int resmisa_heads(int g);
hipError_t launch_resmisa_gather(const sa_problem& p, const sa_tensor& q, const sa_tensor& w, int g, const int32_t* heads,
                                 uint16_t* qa, float* wa, hipStream_t s);

// SA_DEBUG_CHECKS: candidate lists checked for repeated positions (histories of at most
// kCheckMaxPositions) and for entries that are neither -1 nor visible; sets SA_ERR_INDEX.
constexpr int kCheckMaxPositions = 1 << 18;
hipError_t launch_check_indices(const sa_problem& p, const int32_t* idx, Status* status, hipStream_t s);

// Environment switches, read at every call (debugging and tuning only): an integer value,
// or dflt when the variable is unset, empty or not a number.
inline int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    char* end = nullptr;
    const long x = std::strtol(v, &end, 10);
    return (*end == 0 && x >= -(1L << 30) && x <= (1L << 30)) ? (int)x : dflt;
}
inline bool env_flag(const char* name) { return env_int(name, 0) != 0; }

// Host-side planning shared by workspace sizing and launches.
int attn_splits(const sa_problem& p);
bool attn_uses_mla(const sa_problem& p, int dtype);
bool attn_paged_ok(const AttnArgs& a);  // a paged call runs on the LDS latent or the bf16 MHA kernel
size_t attn_partial_bytes(const sa_problem& p);

}  // namespace sa
