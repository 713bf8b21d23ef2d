/*
 * sa.h -- C ABI of libsa.so: content-routed token-sparse attention with a
 * Lightning-Indexer-style selector, for AMD MI355X (gfx950).
 *
 * The path has three steps, each with its own entry point, plus one fused call:
 *   1. sa_indexer_score  proxy score  r[b,i,j] = sum_h w[b,i,h] * ReLU(<q_idx[b,i,h,:], k_idx[b,j,:]>)
 *                        over the visible history of every query row.
 *   2. sa_topk           per-row top-k of those scores with a deterministic
 *                        (score desc, position asc) order; indices in ascending position.
 *   3. sa_sparse_attn    exact softmax attention over the selected rows only, with one
 *                        candidate set shared by all main heads of a query.
 *   sa_select_attend     1 -> 2 -> 3 in one call.
 * Definitions are those of "PaperTrace 2.2 · Fine-grained indexing" (§1.1 and §3.2 for the
 * score, §2.1 eq. (4) and the following paragraphs for the selection, §3.1 for the tie
 * rule and the finiteness check) and "PaperTrace 2.1.1 · Hashing and clustering" (§1.1 for
 * sparse attention over a candidate set intersected with the causal and padding masks,
 * §5.1 for one softmax shared by all candidate pieces).
 *
 * ---- Conventions shared by every entry point ---------------------------------------
 * Memory.  Every pointer argument is DEVICE memory on the current HIP device unless
 *   stated otherwise.  The caller owns every buffer, including the workspace; the library
 *   never allocates or frees memory and keeps no global state.  All work is enqueued on
 *   `stream` (a hipStream_t passed as void*; NULL = the default stream) and is
 *   asynchronous: buffers must stay valid until the stream reaches the work.
 * Errors.  Argument errors are detected on the host before anything is launched and are
 *   returned synchronously (SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE).  A
 *   launch failure returns SA_ERR_HIP.  Non-finite visible scores (from non-finite index
 *   inputs) are detected on the device and recorded in a status word in the workspace,
 *   read by sa_device_status(); outputs of such a row are unspecified.
 * Positions and masks.  Query row i of batch b sits at absolute position
 *   q_pos(b,i) = q_pos0[b] + i.  History position j is visible to that row iff
 *   j < kv_len[b] and, when causal, j <= q_pos(b,i) (a query sees itself).  A query row is
 *   valid iff q_pos(b,i) < kv_len[b]; an invalid (padded) row gets idx all -1, O = 0 and
 *   LSE = -inf.
 * Tensors.  An sa_tensor is a strided view whose last dimension is contiguous:
 *   element (i0, i1, i2, d) lives at data + i0*s0 + i1*s1 + i2*s2 + d (strides in
 *   ELEMENTS).  The data pointer must be 16-byte aligned and every stride times the element
 *   size a multiple of 16 bytes.  Dimension order per tensor is given at each argument.
 * Dtypes.  SA_F32, SA_BF16 (bit pattern of the upper half of an f32) and SA_FP8_E4M3
 *   (OCP e4m3fn: bias 7, no infinities, 0x7f/0xff are NaN, max 448).
 * Environment (read at every call):
 *   SA_DEBUG_CHECKS=1  before the attention of sa_sparse_attn, sa_sparse_attn_paged and
 *                      sa_select_attend, a check kernel reads every candidate list and sets
 *                      SA_ERR_INDEX in the status word when a list holds the same position
 *                      twice (duplicates must be removed before the softmax: "PaperTrace 2.2",
 *                      §2.1, and "PaperTrace 2.1.1", §5.1) or an entry other than -1 that is
 *                      not visible to its row (such entries are otherwise skipped).  Repeats
 *                      are checked for histories of at most 2^19 positions.
 *   SA_FORCE_UNFUSED=1 sa_select and sa_select_attend store score rows and run the separate
 *                      top-k (in row slices that fit the same workspace) instead of the
 *                      streaming selection; the result is the same.
 *   SA_SPLITS=n        candidate splits of the latent-head attention (clamped to what the
 *                      kernel takes); workspace sizes depend on it, so size and call with
 *                      the same setting.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 2

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1, /* null pointer, bad size or stride, inconsistent dims */
    SA_ERR_UNSUPPORTED = 2, /* valid but not implemented: dtype combination or head size */
    SA_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than sa_workspace_bytes() */
    SA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
    SA_ERR_NONFINITE = 5,   /* device side: a visible score was NaN or infinite */
    SA_ERR_INDEX = 6        /* device side, SA_DEBUG_CHECKS=1 only: a candidate list holds a
                               position twice, or an entry that is neither -1 nor visible */
} sa_status;

typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1, SA_FP8_E4M3 = 2 } sa_dtype;

typedef enum sa_op {
    SA_OP_INDEXER_SCORE = 0,
    SA_OP_TOPK = 1,
    SA_OP_SPARSE_ATTN = 2,
    SA_OP_SELECT_ATTEND = 3,
    SA_OP_SPARSE_ATTN_PAGED = 4,
    SA_OP_SELECT = 5
} sa_op;

typedef struct sa_tensor {
    void* data;       /* device pointer, 16-byte aligned */
    int32_t dtype;    /* sa_dtype */
    int64_t s0, s1, s2; /* element strides of the three leading dimensions */
} sa_tensor;

typedef struct sa_problem {
    int32_t B;      /* batch */
    int32_t n_q;    /* query rows per batch */
    int32_t n_kv;   /* history capacity per batch (rows of k_idx / K / V) */
    int32_t Hq;     /* main query heads */
    int32_t Hkv;    /* main key/value heads; Hq % Hkv == 0 (grouped sharing) */
    int32_t d_qk;   /* main query/key head width */
    int32_t d_v;    /* main value head width */
    int32_t Hidx;   /* index heads */
    int32_t d_idx;  /* index head width */
    int32_t k;      /* selection budget per query row, >= 1 */
    int32_t causal; /* 1: j visible only if j <= q_pos(b,i); 0: the whole valid history */
    const int32_t* kv_len; /* device [B], valid history length per batch, <= n_kv; NULL = n_kv */
    const int32_t* q_pos0; /* device [B], absolute position of query row 0; NULL = 0 */
    float scale;    /* softmax logit scale; 0 selects 1/sqrt(d_qk) */
} sa_problem;

/*
 * sa_indexer_score -- the proxy score of every (query row, history position).
 * "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §3.2: per-query index heads, one
 * index key per token shared by all heads, query-dependent head weights, ReLU matching.
 *   q_idx  [B, n_q, Hidx, d_idx]  f32 or bf16      (s0 = batch, s1 = row, s2 = head)
 *   k_idx  [B, n_kv, d_idx]       f32, bf16, e4m3  (s0 = batch, s1 = position; s2 unused)
 *   w      [B, n_q, Hidx]         f32              (s0 = batch, s1 = row; s2 unused)
 *   scores [B, n_q, n_kv] f32, contiguous: scores[(b*n_q + i)*n_kv + j]; -inf where j is
 *          not visible (and on every position of an invalid row).
 * Accumulation is fp32 over exact bf16 products (e4m3 widens exactly to bf16).  The
 * reduction order does not depend on j, so byte-identical index keys score bit-identically.
 */
sa_status sa_indexer_score(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w,
                           float* scores, void* stream);

/*
 * sa_topk -- per-row selection.  "PaperTrace 2.2 · Fine-grained indexing", §2.1 eq. (4),
 * the causal-prefill paragraph (rows with fewer than k visible positions return all of
 * them and mark the other slots invalid) and §3.1 (lexicographic (score, index) order).
 *   scores  f32, row (b,i) at scores + (b*n_q + i)*row_stride; only visible entries are read.
 *   idx     [B, n_q, k] int32, contiguous: the first min(k, |visible|) positions in
 *           (score desc, position asc) order, written in ascending position, then -1.
 *   vals    [B, n_q, k] f32 or NULL: the score of each idx entry (-inf for -1 slots).
 *   ws      workspace of at least sa_workspace_bytes(p, SA_OP_TOPK) bytes, 256-byte
 *           aligned, zero-filled by the caller once after allocation (it carries the
 *           device status word between calls).
 * A NaN or infinite visible score sets SA_ERR_NONFINITE in the status word.
 */
sa_status sa_topk(const sa_problem* p, const float* scores, int64_t row_stride, int32_t* idx, float* vals,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * sa_select -- score and select in one call: the output of sa_indexer_score followed by
 * sa_topk (idx as there, bit for bit), without the scores.  "PaperTrace 2.2 · Fine-grained
 * indexing", §2.1: the selector works through the history slice by slice, keeps local
 * candidates and merges them down to k, which gives the global top-k; the full score
 * matrix is never materialised.  This streaming form runs when the index queries are bf16,
 * the index keys bf16 or e4m3, Hidx is 16, 32 or 64, d_idx 64 or 128 and there are enough
 * query rows (at least 512 blocks of 512 / Hidx rows); there each row's candidates above a
 * running threshold are kept in the workspace (about 2k + 128 entries per row of a
 * bounded number of rows in flight) and cut back to k when full.  Other calls store the
 * visible scores of each row in the workspace and select from them.
 *   q_idx, k_idx, w   as for sa_indexer_score
 *   idx               [B, n_q, k] int32, contiguous, as for sa_topk
 *   ws                sa_workspace_bytes(p, SA_OP_SELECT) bytes, 256-byte aligned,
 *                     zero-filled once after allocation (status word: non-finite index
 *                     inputs of valid rows or visible keys set SA_ERR_NONFINITE).
 * The workspace size depends on the shape only: for a shape that takes the streaming form
 * but f32 index inputs, the rows are scored and selected in slices through the same space.
 */
sa_status sa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, int32_t* idx, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * sa_sparse_attn -- exact softmax attention over the selected history rows.
 * "PaperTrace 2.1.1 · Hashing and clustering", §1.1 eq. (1): logits, mask, softmax and
 * value aggregation only over the candidate set; §5.1: every piece of the set shares one
 * row maximum and exp-sum (split pieces are merged by log-sum-exp).
 *   Q [B, Hq, n_q, d_qk], K [B, Hkv, n_kv, d_qk], V [B, Hkv, n_kv, d_v]   (s0 = batch,
 *      s1 = head, s2 = row).  Q, K, V and O share one dtype, f32 or bf16.  V may alias K
 *      (latent layout: V = the first d_v columns of each K row, same strides).
 *   idx [B, n_q, k] int32, contiguous; entries that are -1, out of range or not visible
 *      are ignored (never read).  Valid entries must be unique (a duplicate would count
 *      twice in the softmax); their order does not matter.  K/V rows that no entry selects
 *      are never read.  The multi-head kernel for many query rows (bf16, d_qk = d_v = 128)
 *      computes blocks of 64 query rows of a batch together: a row selected by any query
 *      row of the block is read for the whole block and enters the other rows' value
 *      product with weight 0, so a non-finite value in a SELECTED K/V row can reach the
 *      outputs of other rows of that block.
 *   O   [B, Hq, n_q, d_v] output; query head h reads key/value head h / (Hq / Hkv).
 *   lse [B, Hq, n_q] f32 or NULL: natural-log log-sum-exp of the scaled logits
 *      (-inf when a row has no valid entry; then O = 0).
 *   ws  workspace of at least sa_workspace_bytes(p, SA_OP_SPARSE_ATTN) bytes.
 * Logits and softmax statistics are fp32; probabilities are rounded to the input dtype for
 * the value product on the matrix-core path.
 */
sa_status sa_sparse_attn(const sa_problem* p, sa_tensor Q, sa_tensor K, sa_tensor V, const int32_t* idx,
                         sa_tensor O, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * sa_sparse_attn_paged -- sa_sparse_attn over K/V held in fixed-size pages.
 * "PaperTrace 2.2 · Fine-grained indexing", §2.1 (the gather of the main KV: the selected
 * logical positions go through the block table to physical rows before the attention
 * reads them) and §3.1 (the block table among the objects of the sparse-attention call).
 * The result is that of sa_sparse_attn on the logical K/V in which position j of batch b
 * is physical row  block_table[b*bt_stride + j/page_size]*page_size + j%page_size  of the pools.
 *   K, V        page pools: element (head h, physical row r, column c) at data + h*s1 +
 *               r*s2 + c (s0 is not used); pool_rows rows per head; V may alias K as above.
 *   pool_rows   rows in the pools (a whole number of pages is expected; a page that does
 *               not fit entirely is never read).
 *   block_table int32, device; row b holds the page numbers of batch b's logical pages
 *               0 .. ceil(n_kv/page_size) - 1; bt_stride >= that count.  Only pages that
 *               hold a visible selected position are read.  A page number outside
 *               [0, pool_rows/page_size) skips the candidate (as an idx entry of -1 would).
 *   page_size   a power of two, 1 .. 65536.
 *   ws          workspace of at least sa_workspace_bytes(p, SA_OP_SPARSE_ATTN_PAGED) bytes
 *               (it holds the translated candidate rows of the multi-head kernel).
 * Q, idx, O, lse and the dtypes are as for sa_sparse_attn.  The call is supported on
 * the two matrix-core/vector kernels: bf16 latent (d_qk 576, d_v 512, V aliasing K,
 * 32/64/128 query heads per key head, pool_rows * row stride below 2^31 bytes) and bf16
 * multi-head with Hq == Hkv and d_qk == d_v in {64, 128, 256} (k a multiple of 4, fewer
 * than 2^24 pool rows); other shapes return SA_ERR_UNSUPPORTED.
 */
sa_status sa_sparse_attn_paged(const sa_problem* p, sa_tensor Q, sa_tensor K, sa_tensor V, int64_t pool_rows,
                               const int32_t* block_table, int64_t bt_stride, int page_size, const int32_t* idx,
                               sa_tensor O, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * sa_select_attend -- sa_select, then sa_sparse_attn, in one call; arguments as in those
 * entry points.  idx_out [B, n_q, k] int32 receives the selection if not NULL.
 * ws must hold sa_workspace_bytes(p, SA_OP_SELECT_ATTEND) bytes, zero-filled once (status
 * word); it includes the space of the selection (candidate lists, or the visible scores
 * where the streaming form does not apply).
 */
sa_status sa_select_attend(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, sa_tensor Q,
                           sa_tensor K, sa_tensor V, int32_t* idx_out, sa_tensor O, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * sa_select_attend_noalloc -- sa_select_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid it): the
 * same kernels and results, with the workspace replaced by a fixed 64 MiB array of device
 * memory inside the library.  Each GPU the library runs on holds its own copy of that array
 * until the process ends.  Nothing is allocated or freed by the call.
 *   arguments as for sa_select_attend, without ws / ws_bytes;
 *   status  device pointer to a zero-filled, 256-byte aligned block of 256 bytes, or NULL:
 *           receives the status word (SA_ERR_NONFINITE), read and cleared by
 *           sa_device_status(status, stream); NULL = not reported.
 * Problems whose sa_workspace_bytes(p, SA_OP_SELECT_ATTEND) exceeds 64 MiB (for example
 * long prefills) return SA_ERR_WORKSPACE before anything is launched.  All calls on one GPU
 * share its array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give undefined results; calls ordered on one stream are safe.
 */
sa_status sa_select_attend_noalloc(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, sa_tensor Q,
                                   sa_tensor K, sa_tensor V, int32_t* idx_out, sa_tensor O, float* lse,
                                   uint32_t* status, void* stream);

/*
 * sa_select_attend_grouped -- grouped candidate sets.  "PaperTrace 2.2 · Fine-grained
 * indexing", §2 eq. (5) and the paragraphs around it (shared versus per-head candidates):
 * the Hq main heads form G groups, each with its own selector, S_{t,g} = TopK(Agg over the
 * group's heads of r, k_g); G = 1 is the shared set of sa_select_attend.  Reading where the
 * pages leave the step open: heads are grouped contiguously and in equal numbers, the
 * index heads are grouped the same way (Hidx / G per group, a multiple of 4 when G > 1),
 * Agg is the indexer's own weighted ReLU sum over the group's index heads, k_g = k for
 * every group, and group g's Hq / G query heads attend over S_{t,g} with the same tie rule.
 * The key/value heads split into G groups as well (Hkv a multiple of G), or all groups
 * share the single key/value head (Hkv = 1, the latent layout).
 *   arguments as for sa_select_attend, the group problem (Hq / G, Hkv / G or 1, Hidx / G)
 *   supported by sa_sparse_attn;
 *   idx_out [G, B, n_q, k] int32 (16-byte aligned) or NULL: group g's selection at
 *           idx_out + g*B*n_q*k;
 *   ws      sa_grouped_workspace_bytes(p, groups) bytes, zero-filled once (status word).
 * The groups run one after another on the stream, each as select (sa_select's streaming
 * form where it applies, so no score rows are stored) and attend.
 */
sa_status sa_select_attend_grouped(const sa_problem* p, int groups, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w,
                                   sa_tensor Q, sa_tensor K, sa_tensor V, int32_t* idx_out, sa_tensor O,
                                   float* lse, void* ws, size_t ws_bytes, void* stream);
/* Workspace bytes of sa_select_attend_grouped; 0 when p or groups is not accepted. */
size_t sa_grouped_workspace_bytes(const sa_problem* p, int groups);

/* Workspace bytes needed by operation `op` (an sa_op) for problem p; 0 for a malformed p. */
size_t sa_workspace_bytes(const sa_problem* p, int op);

/*
 * Hierarchical selection.  "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the HISA paragraphs
 * (coarse-to-fine search domain, cost O(B d_c + k_b b d_r), conditional recall eq. (7)):
 * the history is cut into blocks of `blk` positions, each block is scored through a
 * representative key, the k_blocks best blocks are kept and the token scores run only
 * inside them.  Readings where the pages leave the step open: a block's representative is
 * the mean of its blk index keys rounded to bf16 and is scored with the indexer's own
 * formula (d_c = d_idx); only complete blocks inside a row's visible prefix compete (block
 * B is a candidate of row (b, i) iff (B + 1) blk <= L(b, i)); the open block
 * [floor(L / blk) blk, L) is always a token candidate; blocks and tokens are both ranked
 * by (score desc, position asc).
 *
 * sa_block_means -- the representatives, kept with the index keys (a coarse index built
 * once per completed block, not per selection).
 *   k_idx  [B, n_kv, d_idx]  f32, bf16 or e4m3 (as for sa_indexer_score), d_idx <= 256
 *   blk    16, 32, 64, 128 or 256
 *   kbar   [B, n_kv / blk, d_idx] bf16 bit patterns, contiguous, caller-owned device memory;
 *          block B of batch b = positions [B blk, (B + 1) blk).  Blocks past kv_len hold
 *          means of padding and are never candidates.
 */
sa_status sa_block_means(const sa_problem* p, sa_tensor k_idx, int blk, uint16_t* kbar, void* stream);

/* Workspace bytes of sa_hisa_select; 0 for malformed arguments. */
size_t sa_hisa_workspace_bytes(const sa_problem* p, int blk, int k_blocks);

/*
 * sa_hisa_select -- block top-k_blocks over the representatives, then token top-k over
 * the kept blocks and the open block.
 *   q_idx, k_idx, w   as for sa_indexer_score; q_idx and w must have s0 = n_q * s1 (rows of
 *                     all batches equally spaced)
 *   kbar              from sa_block_means with the same k_idx and blk
 *   k_blocks          >= 1, (k_blocks + 1) * blk <= 32768
 *   idx               [B, n_q, k] int32, contiguous: like sa_topk, the selected positions in
 *                     ascending order, then -1
 *   blocks            [B, n_q, k_blocks] int32, contiguous, or NULL: the kept blocks of each
 *                     row in ascending order, then -1 (the coarse candidates, so that a miss
 *                     can be traced to the block or the token stage)
 *   ws                sa_hisa_workspace_bytes(p, blk, k_blocks) bytes, 256-byte aligned,
 *                     zero-filled once after allocation (its first word is the status word
 *                     read by sa_device_status: non-finite scores set SA_ERR_NONFINITE).
 */
sa_status sa_hisa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, const uint16_t* kbar,
                         int blk, int k_blocks, int32_t* idx, int32_t* blocks, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * Active index heads.  "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the MISA paragraphs: each
 * query row keeps g of its Hidx index heads and its score sums only those heads.  The heads
 * are chosen from the block representatives of sa_block_means: routing score of head h =
 * |w_h| times the mean over the row's complete visible blocks B of ReLU(<q_h, kbar_B>)
 * (0 for a row without a complete visible block); the g best by (routing score desc, head
 * asc) are kept.  Then the token scores sum the kept heads only and the top-k is taken as
 * by sa_topk.
 *
 * sa_misa_select
 *   q_idx, k_idx, w   as for sa_indexer_score; q_idx bf16, Hidx 16, 32 or 64, d_idx 64 or 128
 *   kbar, blk         from sa_block_means with the same k_idx
 *   g                 active heads per row, 1 <= g <= Hidx
 *   idx               [B, n_q, k] int32, contiguous, as for sa_topk
 *   heads             [B, n_q, g] int32, contiguous, or NULL: the active heads, ascending
 *   ws                sa_misa_workspace_bytes(p, blk, g) bytes, 256-byte aligned,
 *                     zero-filled once after allocation (status word as for sa_topk; it
 *                     includes the token selection's space, as for sa_select with g index
 *                     heads: candidate lists for many query rows, score rows otherwise).
 */
sa_status sa_misa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, const uint16_t* kbar,
                         int blk, int g, int32_t* idx, int32_t* heads, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of sa_misa_select; 0 for malformed or unsupported arguments. */
size_t sa_misa_workspace_bytes(const sa_problem* p, int blk, int g);

/*
 * Shared linear term plus residual heads (ResMiSA).  "PaperTrace 2.2 · Fine-grained
 * indexing", §2.2, the ResMiSA paragraph: since ReLU(z) = z + ReLU(-z), the heads' linear
 * terms add up to one shared dot product and only some heads keep the non-linear part:
 *     r = <sum_h w_h q_h, k> + sum_{h active} w_h ReLU(-<q_h, k>),
 * which equals the indexer's score when every head is active.  Reading where the pages
 * leave the step open: the active heads are those of sa_misa_select's routing (same kbar,
 * blk and g), so an inactive head contributes its linear term w_h <q_h, k> instead of
 * nothing; the top-k is taken as by sa_topk.  The shared query is formed in fp32 and enters
 * the matrix cores as three exact bf16 parts, so the score keeps fp32 precision.
 * sa_resmisa_select
 *   arguments as for sa_misa_select; 1 <= g <= min(Hidx, 58)
 *   idx    [B, n_q, k] int32, contiguous, as for sa_topk
 *   heads  [B, n_q, g] int32 or NULL: the residual heads, ascending
 *   ws     sa_resmisa_workspace_bytes(p, blk, g) bytes, 256-byte aligned, zero-filled once
 *          after allocation (status word).
 */
sa_status sa_resmisa_select(const sa_problem* p, sa_tensor q_idx, sa_tensor k_idx, sa_tensor w, const uint16_t* kbar,
                            int blk, int g, int32_t* idx, int32_t* heads, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of sa_resmisa_select; 0 for malformed or unsupported arguments. */
size_t sa_resmisa_workspace_bytes(const sa_problem* p, int blk, int g);

/* Synchronises `stream`, returns the status word accumulated in ws by earlier calls
 * (SA_OK or SA_ERR_NONFINITE) and clears it.  ws is a host-visible pointer to device
 * memory as passed to the other calls. */
sa_status sa_device_status(void* ws, void* stream);

/* Static, human-readable name of a status code. */
const char* sa_status_str(sa_status s);

/* SA_ABI_VERSION of the loaded library. */
int sa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
