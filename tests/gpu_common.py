"""Shared machinery of the GPU parity tests: run the C-ABI entry points on a workload and
compute the matching oracle results on the same bytes."""
import numpy as np
import torch

import sa_synth
import token_selector_gather_amd as sa
from token_selector_gather_amd.inputs import device_workload
from tests.device_inputs import empty_outputs
from oracle import oracle as orc

_cache = {}


def workload(key, **kw):
    if key not in _cache:
        _cache[key] = sa_synth.make_config(**kw)
    return _cache[key]


def decode_f64(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return sa_synth.bf16_to_f32(a).astype(np.float64)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise TypeError(a.dtype)


def score_tolerance(W, rows):
    """Per-entry bound on |r_gpu - r_exact| for fp32 accumulation of d_idx products per head
    and Hidx weighted heads: 2 (d_idx + Hidx + 2) 2^-24 sum_h |w_h| sum_d |q_hd k_d|."""
    q = decode_f64(W["q_idx"])
    k = decode_f64(W["k_idx"])
    w = np.abs(W["w"].astype(np.float64))
    n = W["d_idx"] + W["Hidx"] + 2
    out = np.empty((len(rows), W["n_kv"]))
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        u = (w[b, i][:, None] * np.abs(q[b, i])).sum(0)
        out[r] = 2 * n * 2.0 ** -24 * (np.abs(k[b]) @ u)
    return out


def out_dtype(W):
    return torch.float32 if W["main_dtype"] == sa_synth.F32 else torch.bfloat16


def attn_tol(W):
    return (1e-5, 1e-5) if W["main_dtype"] == sa_synth.F32 else (2e-2, 1e-3)


def gpu_scores(W):
    P, d = device_workload(W, with_main=False)
    sc = torch.full((W["B"], W["n_q"], W["n_kv"]), float("nan"), dtype=torch.float32, device="cuda")
    sa.sa_indexer_score(P, d["q_idx"], d["k_idx"], d["w"], sc)
    torch.cuda.synchronize()
    return sc


def gpu_topk(W, scores):
    P, d = device_workload(W, with_main=False)
    ws = sa.workspace(P, sa.SA_OP_TOPK)
    idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    vals = torch.full((W["B"], W["n_q"], W["k"]), float("nan"), dtype=torch.float32, device="cuda")
    sa.sa_topk(P, scores, W["n_kv"], idx, vals, ws)
    st = sa.sa_device_status(ws)
    return idx.cpu().numpy(), vals.cpu().numpy(), st


def gpu_sparse_attn(W, idx_np):
    P, d = device_workload(W)
    O, lse, _ = empty_outputs(W, out_dtype(W))
    ws = sa.workspace(P, sa.SA_OP_SPARSE_ATTN)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    sa.sa_sparse_attn(P, d["Q"], d["K"], d["V"], idx, O, lse, ws)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), lse.cpu().numpy()


def gpu_select_attend(W, want_idx=True):
    P, d = device_workload(W)
    O, lse, idx = empty_outputs(W, out_dtype(W))
    ws = sa.workspace(P, sa.SA_OP_SELECT_ATTEND)
    sa.sa_select_attend(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx if want_idx else None,
                        O, lse, ws)
    st = sa.sa_device_status(ws)
    return idx.cpu().numpy(), O.float().cpu().numpy(), lse.cpu().numpy(), st


def rows_of(O, lse, W, rows):
    """Gather [B,Hq,n_q,*] GPU outputs into the oracle's [rows, Hq, *] order."""
    b = rows // W["n_q"]
    i = rows % W["n_q"]
    return O[b, :, i, :], lse[b, :, i]


def compare_attention(W, rows, O_gpu, lse_gpu, O_or, lse_or):
    tol_o, tol_l = attn_tol(W)
    Og, Lg = rows_of(O_gpu, lse_gpu, W, rows)
    assert np.isfinite(Og).all()
    err_o = float(np.max(np.abs(Og - O_or))) if Og.size else 0.0
    fin = np.isfinite(lse_or)
    assert np.array_equal(fin, np.isfinite(Lg)), "LSE finiteness differs"
    assert (Lg[~fin] == -np.inf).all()
    err_l = float(np.max(np.abs(Lg[fin] - lse_or[fin]))) if fin.any() else 0.0
    assert err_o <= tol_o, ("O max-abs error", err_o, tol_o)
    assert err_l <= tol_l, ("LSE max-abs error", err_l, tol_l)
    return err_o, err_l


def sample_rows(W, n_each=32, n_rand=64, seed=0):
    """First and last rows of every batch plus random rows (stratified sample)."""
    B, nq = W["B"], W["n_q"]
    rows = set()
    for b in range(B):
        rows.update(range(b * nq, b * nq + min(n_each, nq)))
        rows.update(range(b * nq + max(0, nq - n_each), (b + 1) * nq))
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, B * nq, size=n_rand).tolist())
    return np.array(sorted(rows), dtype=np.int32)


def stratified_rows(W, n_first=64, n_last=64, n_rand=384, seed=0):
    """The first n_first and last n_last valid query rows of the flattened batch plus n_rand
    other valid rows drawn at random: the stratified sample for workloads whose every row
    the oracle cannot score in a test's time."""
    from tests.checker import visible_len
    B, nq = W["B"], W["n_q"]
    valid = np.array([r for r in range(B * nq) if visible_len(W, r // nq, r % nq) > 0], dtype=np.int64)
    if valid.size <= n_first + n_last + n_rand:
        return valid.astype(np.int32)
    ends = np.concatenate([valid[:n_first], valid[-n_last:]])
    rest = np.setdiff1d(valid, ends)
    pick = np.random.default_rng(seed).choice(rest, size=n_rand, replace=False)
    return np.sort(np.concatenate([ends, pick])).astype(np.int32)


def full_check(W, rows=None, tie_groups=None, check_sparse=True, say=None):
    """End-to-end select+attend against the oracle on `rows` (default: all rows), plus the
    attention kernel alone on the oracle's own candidate sets."""
    from tests.checker import check_index_rows
    if rows is None:
        rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    say = say or (lambda x: None)
    idx, O, lse, st = gpu_select_attend(W)
    assert st == sa.SA_OK, sa.sa_status_str(st)
    idx_r = idx.reshape(-1, W["k"])[rows]
    say("oracle scores and selection")
    ref_sc = orc.scores(W, rows)
    ref_idx, sk, skp1, nsel = orc.select(W, ref_sc, rows)
    stats = check_index_rows(W, rows, idx_r, ref_sc, ref_idx, sk, tie_groups=tie_groups)
    say("oracle attention on the GPU's sets")
    O_or, lse_or = orc.attend(W, idx_r, rows)
    errs = compare_attention(W, rows, O, lse, O_or, lse_or)
    errs_sparse = (None, None)
    if check_sparse:
        say("attention on the oracle's sets")
        full = np.full((W["B"] * W["n_q"], W["k"]), -1, dtype=np.int32)
        full[rows] = ref_idx
        O2, lse2 = gpu_sparse_attn(W, full.reshape(W["B"], W["n_q"], W["k"]))
        O_or2, lse_or2 = orc.attend(W, ref_idx, rows)
        errs_sparse = compare_attention(W, rows, O2, lse2, O_or2, lse_or2)
    return dict(stats, err_o=errs[0], err_lse=errs[1], err_o_sparse=errs_sparse[0], idx=idx, ref_idx=ref_idx,
                rows=rows)


def route_tolerance(W, kbar, rows):
    """Bound on |routing score (GPU) - routing score (oracle)| per row."""
    kb = decode_f64(kbar)
    n = W["d_idx"] + 8
    out = np.empty(len(rows))
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        q = decode_f64(W["q_idx"][b, i])
        a = np.abs(q) @ np.abs(kb[b]).T  # [H, nb]
        out[r] = 2 * n * 2.0 ** -24 * (np.abs(W["w"][b, i]) * a.max(axis=1)).max() + 1e-30
    return out
