"""ctypes driver for the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark; never by the library.

Storage dtypes are inferred from numpy arrays: float32 -> f32, uint16 -> bf16 bit
patterns, uint8 -> OCP FP8 e4m3fn codes.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, E4M3 = 0, 1, 2


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "n_q", "n_kv", "Hq", "Hkv", "d_qk", "d_v", "Hidx", "d_idx", "k", "causal")] + [
        ("scale", ctypes.c_double),
        ("kv_len", ctypes.c_void_p),
        ("q_pos0", ctypes.c_void_p),
        ("pos_of_slot", ctypes.c_void_p),
    ]


class _View(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("s0", ctypes.c_int64), ("s1", ctypes.c_int64), ("s2", ctypes.c_int64)]


def build(force=False):
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, src, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P, V = ctypes.POINTER(_Problem), _View
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.or_scores.argtypes = [P, V, V, V, i64, vp, vp, i32]
        L.or_scores.restype = i32
        L.or_select.argtypes = [P, vp, i64, vp, vp, vp, vp, vp, i32]
        L.or_select.restype = None
        L.or_attend.argtypes = [P, V, V, V, vp, i64, i64, vp, vp, vp, i32]
        L.or_attend.restype = i32
        L.or_count_visible.argtypes = [P]
        L.or_count_visible.restype = ctypes.c_int64
        L.or_decode_one.argtypes = [i32, ctypes.c_uint32]
        L.or_decode_one.restype = ctypes.c_double
        _lib = L
    return _lib


def threads():
    """Worker threads: the CPUs this process may run on, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, min(64, n))


def _dtype_code(a):
    return {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): E4M3}[a.dtype]


def _view(a, ncols=None):
    """Strided view of a numpy array whose last dimension is contiguous; 2-, 3- and
    4-d arrays map to (s0, s1, s2) element strides of their leading dimensions."""
    assert a.strides[-1] == a.itemsize, "last dimension must be contiguous"
    st = [s // a.itemsize for s in a.strides[:-1]]
    st = st + [0] * (3 - len(st))
    return _View(a.ctypes.data, _dtype_code(a), st[0], st[1], st[2])


class Problem:
    """Keeps the ctypes problem struct and the host arrays it points into alive."""

    def __init__(self, W, pos_of_slot=None, k=None, causal=None, scale=None):
        self.kv_len = np.ascontiguousarray(W["kv_len"], dtype=np.int32)
        self.q_pos0 = np.ascontiguousarray(W["q_pos0"], dtype=np.int32)
        self.pos = None if pos_of_slot is None else np.ascontiguousarray(pos_of_slot, dtype=np.int32)
        s = W["scale"] if scale is None else scale
        self.p = _Problem(W["B"], W["n_q"], W["n_kv"], W["Hq"], W["Hkv"], W["d_qk"], W["d_v"], W["Hidx"],
                          W["d_idx"], W["k"] if k is None else k, W["causal"] if causal is None else causal,
                          float(s), self.kv_len.ctypes.data, self.q_pos0.ctypes.data,
                          None if self.pos is None else self.pos.ctypes.data)
        self.k = self.p.k


def _rows(W, rows):
    if rows is None:
        rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    return np.ascontiguousarray(rows, dtype=np.int32)


def scores(W, rows=None, pos_of_slot=None, k_idx=None):
    """fp64 indexer scores [len(rows), n_kv]; -inf where not visible."""
    P = Problem(W, pos_of_slot)
    rows = _rows(W, rows)
    q, kk, w = W["q_idx"], W["k_idx"] if k_idx is None else k_idx, W["w"]
    out = np.empty((rows.size, W["n_kv"]), dtype=np.float64)
    rc = lib().or_scores(ctypes.byref(P.p), _view(q), _view(kk), _view(w), rows.size, rows.ctypes.data,
                         out.ctypes.data, threads())
    if rc != 0:
        raise ValueError("oracle: non-finite index input")
    return out


def select(W, sc, rows=None, pos_of_slot=None, k=None):
    """Top-k of given fp64 score rows.  Returns (idx int32 [n,k], s_k, s_k+1, n_selected)."""
    P = Problem(W, pos_of_slot, k=k)
    rows = _rows(W, rows)
    sc = np.ascontiguousarray(sc, dtype=np.float64)
    assert sc.shape == (rows.size, W["n_kv"])
    n = rows.size
    idx = np.empty((n, P.k), dtype=np.int32)
    sk, skp1 = np.empty(n), np.empty(n)
    nsel = np.empty(n, dtype=np.int32)
    lib().or_select(ctypes.byref(P.p), sc.ctypes.data, n, rows.ctypes.data, idx.ctypes.data, sk.ctypes.data,
                    skp1.ctypes.data, nsel.ctypes.data, threads())
    return idx, sk, skp1, nsel


def attend(W, idx, rows=None, pos_of_slot=None, Q=None, K=None, V=None, scale=None):
    """fp64 softmax attention of the listed rows over idx ([n, k] slots, -1 skipped).
    Returns (O [n, Hq, d_v], lse [n, Hq])."""
    P = Problem(W, pos_of_slot, k=np.asarray(idx).shape[1], scale=scale)
    rows = _rows(W, rows)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Q = W["Q"] if Q is None else Q
    K = W["K"] if K is None else K
    V = W["V"] if V is None else V
    if V is None:  # latent layout: V is the first d_v columns of each K row
        V = K[..., : W["d_v"]]
    n = rows.size
    O = np.empty((n, W["Hq"], W["d_v"]), dtype=np.float64)
    lse = np.empty((n, W["Hq"]), dtype=np.float64)
    rc = lib().or_attend(ctypes.byref(P.p), _view(Q), _view(K), _view(V), idx.ctypes.data, idx.shape[1], n,
                         rows.ctypes.data, O.ctypes.data, lse.ctypes.data, threads())
    if rc != 0:
        raise ValueError("oracle: non-finite attention input")
    return O, lse


def attend_paged(W, idx, K_pool, V_pool, block_table, page_size, rows=None):
    """attend() over K/V held in pages.  "PaperTrace 2.2 · Fine-grained indexing", §2.1 (the
    gather of the main KV: selected logical positions pass through the block table before
    the attention reads physical rows) and §3.1 (block_table maps logical positions to
    physical pages).  Logical row j of batch b is pool row
    block_table[b, j // page_size] * page_size + j % page_size; K_pool, V_pool are
    [Hkv, pool_rows, d] (V_pool None: the latent layout, V = the first d_v columns of K).
    Reading: a candidate whose page number lies outside the pool is skipped, as a -1 slot.
    The pools are un-paged into the contiguous layout, then attend() runs on it."""
    K_pool = np.asarray(K_pool)
    bt = np.asarray(block_table, dtype=np.int64)
    B, n_kv = W["B"], W["n_kv"]
    pool_pages = K_pool.shape[1] // page_size
    j = np.arange(n_kv)
    page = bt[:, j // page_size]                                   # [B, n_kv]
    ok = (page >= 0) & (page < pool_pages)
    phys = np.where(ok, page * page_size + j % page_size, 0)       # [B, n_kv]
    K = np.ascontiguousarray(K_pool[:, phys].transpose(1, 0, 2, 3))  # [B, Hkv, n_kv, d]
    V = None if V_pool is None else np.ascontiguousarray(np.asarray(V_pool)[:, phys].transpose(1, 0, 2, 3))
    rows_ = _rows(W, rows)
    idx = np.array(idx, dtype=np.int32, copy=True)
    b_of = rows_ // W["n_q"]
    inr = (idx >= 0) & (idx < n_kv)
    bad = inr & ~ok[b_of[:, None], np.clip(idx, 0, n_kv - 1)]
    idx[bad] = -1
    return attend(W, idx, rows_, K=K, V=V)


def group_workload(W, G, g):
    """The problem of group g of G: index heads and query heads [g H/G, (g+1) H/G), the
    key/value heads of the group (or the one shared key/value head)."""
    Hig, Hg = W["Hidx"] // G, W["Hq"] // G
    Wg = dict(W)
    Wg["Hidx"], Wg["Hq"] = Hig, Hg
    Wg["q_idx"] = np.ascontiguousarray(W["q_idx"][:, :, g * Hig:(g + 1) * Hig])
    Wg["w"] = np.ascontiguousarray(W["w"][:, :, g * Hig:(g + 1) * Hig])
    Wg["Q"] = np.ascontiguousarray(W["Q"][:, g * Hg:(g + 1) * Hg])
    if W["Hkv"] > 1:
        Hkg = W["Hkv"] // G
        Wg["Hkv"] = Hkg
        Wg["K"] = np.ascontiguousarray(W["K"][:, g * Hkg:(g + 1) * Hkg])
        if W.get("V") is not None:
            Wg["V"] = np.ascontiguousarray(W["V"][:, g * Hkg:(g + 1) * Hkg])
    return Wg


def select_attend_grouped(W, G, rows=None):
    """Grouped candidate sets, "PaperTrace 2.2 · Fine-grained indexing", §2 eq. (5): the main
    heads form G groups, each with its own selector; S_{t,g} = TopK over the group's
    aggregated scores.  Reading: equal contiguous groups of query heads and of index heads,
    Agg = the indexer's weighted ReLU sum over the group's index heads, k_g = k, and group
    g's query heads attend over S_{t,g}.  Returns idx [G, rows, k], O [rows, Hq, d_v],
    lse [rows, Hq] (query heads in their original order)."""
    rows = _rows(W, rows)
    idx, O, lse = [], [], []
    for g in range(G):
        r = select_attend(group_workload(W, G, g), rows)
        idx.append(r["idx"])
        O.append(r["O"])
        lse.append(r["lse"])
    return np.stack(idx), np.concatenate(O, axis=1), np.concatenate(lse, axis=1)


def count_visible(W, causal=None):
    P = Problem(W, causal=causal)
    return lib().or_count_visible(ctypes.byref(P.p))


def decode(dtype, bits):
    return lib().or_decode_one(dtype, int(bits))


def select_attend(W, rows=None):
    """Full path on the listed rows: scores -> select -> attention."""
    rows = _rows(W, rows)
    sc = scores(W, rows)
    idx, sk, skp1, nsel = select(W, sc, rows)
    O, lse = attend(W, idx, rows)
    return dict(scores=sc, idx=idx, sk=sk, skp1=skp1, nsel=nsel, O=O, lse=lse)


# ------------------------------------------------------------------ hierarchical selection
# "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the HISA paragraphs (coarse-to-fine search
# domain): the history is cut into blocks of b positions, each block is scored through a
# representative, the k_b best blocks are kept, and the token indexer runs only inside
# them; the output keeps the token top-k interface.  Readings (the pages leave these open):
#  * representative of a block = the mean of its b index keys, rounded to bf16 (the
#    precision the kernels score it in), scored with the same weighted-ReLU formula;
#  * only complete blocks inside a row's visible prefix compete (block B of row (b, i) is
#    visible iff (B + 1) b <= L(b, i)); the open block [P b, L), P = floor(L / b), is always
#    a candidate (the pages hand unfinished blocks to a local path);
#  * blocks and tokens are both ranked by (score desc, position asc).

_DEC = {}


def _decode_table(dtype):
    """Value of every bit pattern of a storage dtype, from this oracle's own decoder."""
    if dtype not in _DEC:
        n = 256 if dtype == E4M3 else 65536
        _DEC[dtype] = np.array([decode(dtype, c) for c in range(n)], dtype=np.float64)
    return _DEC[dtype]


def decode_array(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    return _decode_table(_dtype_code(a))[a.astype(np.int64)]


def f64_to_bf16_bits(x):
    """Round-to-nearest-even of fp64 values to bf16 bit patterns (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    y = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits, ties to even
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def block_means(W, blk, batches=None):
    """Block representatives [B, n_kv // blk, d_idx] (or [len(batches), ...]) as bf16 bit
    patterns: the mean of each complete block of blk index keys (fp64 sum of the decoded
    keys, rounded once)."""
    batches = np.arange(W["B"]) if batches is None else np.asarray(batches)
    nb = W["n_kv"] // blk
    out = np.empty((batches.size, nb, W["d_idx"]), dtype=np.uint16)
    for n, b in enumerate(batches):
        k = decode_array(W["k_idx"][b, : nb * blk])
        out[n] = f64_to_bf16_bits(k.reshape(nb, blk, W["d_idx"]).sum(axis=1) / blk)
    return out


def _block_problem(W, blk):
    """The block-level problem: slot B of batch b holds the block's last position, so the
    oracle's visibility test admits exactly the complete blocks inside the visible prefix."""
    nb = W["n_kv"] // blk
    Wb = dict(W)
    Wb["n_kv"] = nb
    ends = np.broadcast_to((np.arange(nb, dtype=np.int32) + 1) * blk - 1, (W["B"], nb))
    return Wb, np.ascontiguousarray(ends, dtype=np.int32)


def hisa_select(W, blk, k_blocks, rows=None, kbar=None):
    """Hierarchical selection of the listed rows.  Returns dict(idx [n, k] positions in
    ascending order, -1 padded; blocks [n, k_blocks] selected block indices ascending, -1
    padded; block_scores [n, n_kv // blk]; bsk / bskp1 the k_b-th and (k_b+1)-th visible
    block scores; ncand candidates per row; csk / cskp1 the k-th and (k+1)-th candidate
    token scores, -inf where they do not exist)."""
    rows = _rows(W, rows)
    if kbar is None:
        kbar = block_means(W, blk)
    Wb, ends = _block_problem(W, blk)
    bsc = scores(Wb, rows, pos_of_slot=ends, k_idx=kbar)
    bidx, bsk, bskp1, _ = select(Wb, bsc, rows, pos_of_slot=ends, k=k_blocks)
    tsc = scores(W, rows)
    L = np.isfinite(tsc).sum(axis=1)  # the visible positions form the prefix [0, L)
    K = W["k"]
    idx = np.full((rows.size, K), -1, dtype=np.int32)
    ncand = np.zeros(rows.size, dtype=np.int64)
    csk, cskp1 = np.full(rows.size, -np.inf), np.full(rows.size, -np.inf)
    for r in range(rows.size):
        P = L[r] // blk
        cand = [np.arange(B * blk, (B + 1) * blk) for B in bidx[r] if B >= 0]
        cand.append(np.arange(P * blk, L[r]))
        pos = np.concatenate(cand).astype(np.int64)
        ncand[r] = pos.size
        if pos.size == 0:
            continue
        s = tsc[r, pos]
        ranked = np.sort(s)[::-1]
        if ranked.size >= K:
            csk[r] = ranked[K - 1]
        if ranked.size > K:
            cskp1[r] = ranked[K]
        order = np.lexsort((pos, -s))[:K]  # score descending, then position ascending
        sel = np.sort(pos[order])
        idx[r, : sel.size] = sel
    return dict(idx=idx, blocks=bidx, block_scores=bsc, bsk=bsk, bskp1=bskp1, token_scores=tsc, ncand=ncand,
                csk=csk, cskp1=cskp1)



# ------------------------------------------------------------------ active index heads
# "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the MISA paragraphs: each query keeps g of its
# G index heads, chosen from the block-averaged index keys (the absolute value of each
# head's weighted ReLU response, averaged over the blocks of the current prefix), and the
# score sums only those heads.  Readings: the blocks are the complete blocks of the visible
# prefix with the bf16 representatives of the hierarchical selection; heads are ranked by
# (routing score desc, head index asc); a row without a complete visible block has all
# routing scores 0 and so keeps heads 0 .. g-1.

def misa_route(W, blk, rows=None, kbar=None):
    """Routing score [n, Hidx] of the listed rows (fp64)."""
    rows = _rows(W, rows)
    if kbar is None:
        kbar = block_means(W, blk)
    kb = decode_array(kbar)
    L = np.isfinite(scores(W, rows)).sum(axis=1)
    out = np.zeros((rows.size, W["Hidx"]))
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        P = int(L[r]) // blk
        if P == 0:
            continue
        q = decode_array(W["q_idx"][b, i])                # [Hidx, d_idx]
        z = np.maximum(q @ kb[b, :P].T, 0.0)              # [Hidx, P]
        out[r] = np.abs(W["w"][b, i].astype(np.float64)) * z.mean(axis=1)
    return out


def misa_heads(route, g):
    """Active heads per row: the g best by (routing score desc, head asc), ascending."""
    H = route.shape[1]
    out = np.empty((route.shape[0], g), dtype=np.int32)
    for r in range(route.shape[0]):
        order = np.lexsort((np.arange(H), -route[r]))[:g]
        out[r] = np.sort(order)
    return out


def misa_select(W, blk, g, rows=None, kbar=None, heads=None):
    """Selection of the listed rows with g active index heads.  Returns dict(idx, heads,
    route, scores, sk, skp1).  `heads` overrides the routing (the GPU's choice, for
    checking the token stage on the same heads)."""
    rows = _rows(W, rows)
    route = misa_route(W, blk, rows, kbar)
    if heads is None:
        heads = misa_heads(route, g)
    b, i = rows // W["n_q"], rows % W["n_q"]
    Wa = dict(W)
    qa = np.stack([W["q_idx"][bb, ii, h] for bb, ii, h in zip(b, i, heads)])  # [n, g, d]
    wa = np.stack([W["w"][bb, ii, h] for bb, ii, h in zip(b, i, heads)])      # [n, g]
    # each listed row as its own batch of one query over its batch's history
    Wa.update(B=rows.size, n_q=1, Hidx=g, q_idx=np.ascontiguousarray(qa[:, None]), w=np.ascontiguousarray(wa[:, None]),
              k_idx=np.ascontiguousarray(W["k_idx"][b]), kv_len=np.asarray(W["kv_len"], np.int32)[b],
              q_pos0=(np.asarray(W["q_pos0"], np.int32)[b] + i).astype(np.int32))
    sc = scores(Wa)
    idx, sk, skp1, _ = select(Wa, sc)
    return dict(idx=idx, heads=heads, route=route, scores=sc, sk=sk, skp1=skp1)


# ------------------------------------------------------------------ shared linear term + residual heads
# "PaperTrace 2.2 · Fine-grained indexing", §2.2, the ResMiSA paragraph: with
# ReLU(z) = z + ReLU(-z), the heads' linear terms add up to ONE shared dot product,
# sum_h w_h <q_h, k> = <sum_h w_h q_h, k>, and the non-linear residual w_h ReLU(-<q_h, k>)
# is computed for some heads only.  Readings: the residual heads are the active heads of
# the MISA routing above (misa_route / misa_heads), so that with every head active the
# score is the indexer's own; the shared query sum_h w_h q_h is formed exactly (fp64).

def resmisa_scores(W, heads, rows=None):
    """ResMiSA scores [n, n_kv] of the listed rows with the given residual heads per row
    ([n, g] head indices; g may be 0): <sum_h w_h q_h, k_j> + sum_{h in heads} w_h
    max(0, -<q_h, k_j>) over the visible j, -inf elsewhere (fp64)."""
    rows = _rows(W, rows)
    L = np.isfinite(scores(W, rows)).sum(axis=1)  # visible prefix [0, L)
    out = np.full((rows.size, W["n_kv"]), -np.inf)
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        n = int(L[r])
        if n == 0:
            continue
        q = decode_array(W["q_idx"][b, i])                  # [Hidx, d_idx]
        w = W["w"][b, i].astype(np.float64)                  # [Hidx]
        k = decode_array(W["k_idx"][b, :n])                  # [n, d_idx]
        qbar = (w[:, None] * q).sum(axis=0)                  # the shared query
        s = k @ qbar
        for h in np.asarray(heads[r], dtype=np.int64):
            s = s + w[h] * np.maximum(0.0, -(k @ q[h]))
        out[r, :n] = s
    return out


def resmisa_select(W, blk, g, rows=None, kbar=None, heads=None):
    """Selection of the listed rows with the shared linear term and g residual heads (the
    MISA routing's active heads unless `heads` overrides them).  Returns dict(idx, heads,
    route, scores, sk, skp1)."""
    rows = _rows(W, rows)
    route = misa_route(W, blk, rows, kbar)
    if heads is None:
        heads = misa_heads(route, g)
    sc = resmisa_scores(W, heads, rows)
    idx, sk, skp1, _ = select(W, sc, rows)
    return dict(idx=idx, heads=heads, route=route, scores=sc, sk=sk, skp1=skp1)
