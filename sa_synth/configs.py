"""The five seeded workload configurations (seed = config id).

Layouts (row-major, last dimension contiguous):
  q_idx [B, n_q, Hidx, d_idx]   index queries, one d_idx vector per index head
  k_idx [B, n_kv, d_idx]        index keys, one vector per token shared by all index heads
  w     [B, n_q, Hidx] f32      query-dependent index-head weights
  Q     [B, Hq, n_q, d_qk]      main queries
  K     [B, Hkv, n_kv, d_qk]    main keys
  V     [B, Hkv, n_kv, d_v]     main values; for the latent (MLA-style) configs V is
                                the first d_v columns of each K row (V is None here)
  kv_len [B] int32, q_pos0 [B] int32: query row i of batch b sits at absolute
  position q_pos0[b] + i; history positions j >= kv_len[b] are padding.

Padding is poisoned: values that would win the selection or dominate the softmax
if a kernel ever read them.
"""
import math

import numpy as np

from . import BF16, E4M3, F32, F64, encode, normal, uniform, bf16_to_f32

# tensor ids of the random streams
T_QIDX, T_KIDX, T_W, T_Q, T_K, T_V, T_LEN, T_CENTRE, T_ASSIGN, T_NEEDLE_POS, T_NEEDLE_JIT = range(1, 12)

CONFIGS = {
    0: dict(name="c0_tiny_prefill_f32", B=1, n_q=256, n_kv=256, Hq=4, Hkv=4, d_qk=64, d_v=64,
            Hidx=4, d_idx=32, k=32, causal=1, main_dtype=F32, qidx_dtype=F32, kidx_dtype=F32,
            main_scale=1.0, mla=False),
    1: dict(name="c1_prefill_bf16_b2_n4096", B=2, n_q=4096, n_kv=4096, Hq=16, Hkv=16, d_qk=128, d_v=128,
            Hidx=8, d_idx=64, k=512, causal=1, main_dtype=BF16, qidx_dtype=BF16, kidx_dtype=BF16,
            main_scale=1.0 / math.sqrt(128.0), mla=False, pad_last=512),
    2: dict(name="c2_mla_prefill_n32768", B=1, n_q=32768, n_kv=32768, Hq=128, Hkv=1, d_qk=576, d_v=512,
            Hidx=64, d_idx=128, k=2048, causal=1, main_dtype=BF16, qidx_dtype=BF16, kidx_dtype=E4M3,
            main_scale=1.0, mla=True),
    3: dict(name="c3_mla_decode_b64_kv65536", B=64, n_q=1, n_kv=65536, Hq=128, Hkv=1, d_qk=576, d_v=512,
            Hidx=64, d_idx=128, k=2048, causal=1, main_dtype=BF16, qidx_dtype=BF16, kidx_dtype=E4M3,
            main_scale=1.0, mla=True, decode=True, len_lo=16384),
    4: dict(name="c4_needle_decode_kv131072", B=1, n_q=8, n_kv=131072, Hq=128, Hkv=1, d_qk=576, d_v=512,
            Hidx=64, d_idx=128, k=1024, causal=0, main_dtype=BF16, qidx_dtype=BF16, kidx_dtype=E4M3,
            main_scale=1.0, mla=True, clusters=512, sigma=0.2, needles=16),
}


def poison_value(dtype):
    """A finite value that would dominate a score or a softmax if it leaked."""
    return {F32: 3.0e4, BF16: 3.0e4, E4M3: 448.0}[dtype]


class Workload(dict):
    """Problem sizes plus host arrays; attribute access for convenience."""

    def __getattr__(self, k):
        try:
            return self[k]
        except KeyError as e:
            raise AttributeError(k) from e


def custom(seed=100, lens=None, q_pos0=None, with_main=True, **kw):
    """A workload with explicit sizes and dtypes (defaults: a small bf16 MHA prefill)."""
    c = dict(name="custom", B=1, n_q=64, n_kv=64, Hq=2, Hkv=2, d_qk=128, d_v=128, Hidx=4, d_idx=64, k=16,
             causal=1, main_dtype=BF16, qidx_dtype=BF16, kidx_dtype=BF16, main_scale=1.0, mla=False)
    c.update(kw)
    return _build(c, cid=-1, seed=seed, lens=lens, q_pos0=q_pos0, with_main=with_main)


def make_config(cid, n=None, n_kv=None, n_q=None, B=None, lens=None, k=None, with_main=True, seed=None):
    """Build config `cid`.  Optional overrides shrink it for oracle-speed parity runs while
    keeping its dtypes, head counts, head dims and structure (padding, ragged lengths)."""
    c = dict(CONFIGS[cid])
    seed = cid if seed is None else seed
    if n is not None:
        c["n_q"] = c["n_kv"] = n
    if n_kv is not None:
        c["n_kv"] = n_kv
    if n_q is not None:
        c["n_q"] = n_q
    if B is not None:
        c["B"] = B
    if k is not None:
        c["k"] = k
    if n is not None and c.get("pad_last"):
        c["pad_last"] = min(c["pad_last"], n // 8)
    return _build(c, cid=cid, seed=seed, lens=lens, q_pos0=None, with_main=with_main)


def _build(c, cid, seed, lens, q_pos0, with_main):
    Bn, nq, nkv = c["B"], c["n_q"], c["n_kv"]
    Hq, Hkv, dqk, dv, Hidx, didx = c["Hq"], c["Hkv"], c["d_qk"], c["d_v"], c["Hidx"], c["d_idx"]
    W = Workload(c)
    W["cid"] = cid
    W["seed"] = seed
    W["scale"] = 1.0 / math.sqrt(dqk)

    # lengths and positions
    if c.get("decode"):
        if lens is None:
            u = uniform(seed, T_LEN, (Bn,), F64)
            lo = min(c["len_lo"], nkv)
            lens = lo + np.floor(u * (nkv - lo + 1)).astype(np.int64)
            lens = np.minimum(lens, nkv)
        kv_len = np.asarray(lens, dtype=np.int32)
        q_pos0 = (kv_len - 1).astype(np.int32)
    else:
        kv_len = np.full((Bn,), nkv, dtype=np.int32)
        if lens is not None:
            kv_len = np.asarray(lens, dtype=np.int32)
        elif c.get("pad_last") and Bn > 1:
            kv_len[1] = nkv - c["pad_last"]
        q_pos0 = np.zeros((Bn,), dtype=np.int32) if q_pos0 is None else np.asarray(q_pos0, dtype=np.int32)
    W["kv_len"] = kv_len
    W["q_pos0"] = q_pos0

    # indexer tensors
    W["q_idx"] = normal(seed, T_QIDX, (Bn, nq, Hidx, didx), c["qidx_dtype"])
    W["w"] = uniform(seed, T_W, (Bn, nq, Hidx), F32)
    if c.get("clusters"):
        W["k_idx"] = _clustered_keys(W, seed)
    else:
        W["k_idx"] = normal(seed, T_KIDX, (Bn, nkv, didx), c["kidx_dtype"])
    pv_idx = encode(np.array([poison_value(c["kidx_dtype"])]), c["kidx_dtype"])[0]
    for b in range(Bn):
        W["k_idx"][b, max(int(kv_len[b]), 0):, :] = pv_idx

    # main attention tensors
    if with_main:
        md, s = c["main_dtype"], c["main_scale"]
        W["Q"] = normal(seed, T_Q, (Bn, Hq, nq, dqk), md, scale=s)
        W["K"] = normal(seed, T_K, (Bn, Hkv, nkv, dqk), md, scale=s)
        W["V"] = None if c["mla"] else normal(seed, T_V, (Bn, Hkv, nkv, dv), md, scale=s)
        pv = encode(np.array([poison_value(md)]), md)[0]
        for b in range(Bn):
            W["K"][b, :, max(int(kv_len[b]), 0):, :] = pv
            if W["V"] is not None:
                W["V"][b, :, max(int(kv_len[b]), 0):, :] = pv
    return W


def _decode_idx_storage(a, dtype):
    if dtype == F32:
        return a.astype(np.float64)
    if dtype == BF16:
        return bf16_to_f32(a).astype(np.float64)
    raise ValueError(dtype)


def _clustered_keys(W, seed):
    """Index keys drawn from Gaussian clusters around unit-norm centres, with planted needles:
    per query, `needles` keys laid along that query's head-weighted index direction
    u = normalise(sum_h w_h q_h) at growing magnitudes.  (Exact-tie groups at the
    selection cutoff need the score and are planted by the tests, not here.)"""
    Bn, nkv, didx, nq = W.B, W.n_kv, W.d_idx, W.n_q
    C, sig = W.clusters, W.sigma
    cen = normal(seed, T_CENTRE, (C, didx), F64)
    cen /= np.linalg.norm(cen, axis=1, keepdims=True)
    assign = np.floor(uniform(seed, T_ASSIGN, (Bn, nkv), F64) * C).astype(np.int64)
    noise = normal(seed, T_KIDX, (Bn, nkv, didx), F64, scale=sig)
    keys = cen[assign] + noise
    # needles
    qd = _decode_idx_storage(W.q_idx, W.qidx_dtype)  # [B, nq, H, d]
    w = W.w.astype(np.float64)
    npos = uniform(seed, T_NEEDLE_POS, (Bn, 4 * nq * W.needles + 64), F64)
    needle_pos = np.zeros((Bn, nq, W.needles), dtype=np.int64)
    for b in range(Bn):
        cand = np.floor(npos[b] * nkv).astype(np.int64)
        _, first = np.unique(cand, return_index=True)
        uniq = cand[np.sort(first)][: nq * W.needles]
        assert uniq.size == nq * W.needles
        needle_pos[b] = uniq.reshape(nq, W.needles)
        for i in range(nq):
            u = (w[b, i, :, None] * qd[b, i]).sum(0)
            u /= np.linalg.norm(u)
            for m in range(W.needles):
                keys[b, needle_pos[b, i, m]] = (6.0 + 0.25 * m) * u * math.sqrt(didx) / 4.0
    W["needle_pos"] = needle_pos
    return encode(keys, W.kidx_dtype)


def paged_layout(seed, B, n_kv, page_size, spare_pages=3):
    """Block table of a paged KV cache: each batch's ceil(n_kv / page_size) logical pages sit
    on distinct pages of one shared pool, chosen by a seeded random permutation, with
    `spare_pages` pages left unused.  Returns (block_table [B, pages] int32, pool_rows)."""
    npg = -(-n_kv // page_size)
    total = B * npg + spare_pages
    perm = np.random.default_rng(seed).permutation(total)[: B * npg].reshape(B, npg)
    return np.ascontiguousarray(perm, dtype=np.int32), total * page_size


def to_pool(X, block_table, page_size, pool_rows, fill):
    """Scatter per-batch rows X [B, H, n_kv, d] into a pool [H, pool_rows, d] along the
    block table; rows no batch uses hold `fill` (a storage value of X's dtype)."""
    B, H, n_kv, d = X.shape
    pool = np.full((H, pool_rows, d), fill, dtype=X.dtype)
    for b in range(B):
        for pg in range(block_table.shape[1]):
            lo = pg * page_size
            if lo >= n_kv:
                break
            hi = min(lo + page_size, n_kv)
            dst = int(block_table[b, pg]) * page_size
            pool[:, dst:dst + hi - lo] = X[b, :, lo:hi]
    return pool
