"""Comparison of GPU results with the oracle.

Index sets (per row): with s_k the oracle's k-th score and eps = 1e-3*|s_k| (or
1e-3*max|r| when s_k == 0), every position scoring above s_k + eps must be selected,
none scoring below s_k - eps may be, the set has min(k, |visible|) members, members are
visible, unique and in ascending order with -1 padding after them; inside each group of
byte-identical index keys the selected members are the lowest positions; and where the
cutoff margin delta_k exceeds twice the largest observed GPU-vs-oracle score error, the
set equals the oracle's exactly ("PaperTrace 2.2 · Fine-grained indexing", §3.1 eq. (9)).
"""
import numpy as np


def visible_len(W, b, i):
    kl = int(W["kv_len"][b])
    qp = int(W["q_pos0"][b]) + i
    if qp < 0 or qp >= kl:
        return 0
    return min(qp + 1, kl) if W["causal"] else kl


def check_index_rows(W, rows, gpu_idx, or_scores, or_idx, or_sk, gpu_scores=None, tie_groups=None):
    """gpu_idx: [len(rows), k] int32.  or_scores: [len(rows), n_kv] fp64 (−inf invisible).
    Returns a dict of statistics; raises AssertionError on a violation."""
    k = W["k"]
    stats = dict(rows=len(rows), exact_rows=0, band_rows=0, max_score_err=0.0)
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        L = visible_len(W, b, i)
        g = gpu_idx[r]
        m = min(k, L)
        sel = g[g >= 0]
        assert sel.size == m, (row, sel.size, m)
        assert (g[m:] == -1).all(), (row, "padding")
        assert np.all(np.diff(sel) > 0), (row, "not ascending / not unique")
        if m == 0:
            continue
        assert sel.max() < L and sel.min() >= 0, (row, "invisible index")
        sc = or_scores[r]
        sk = or_sk[r]
        mx = np.max(np.abs(sc[:L]))
        eps = 1e-3 * abs(sk) if sk != 0 else 1e-3 * mx
        must = np.where(sc[:L] > sk + eps)[0]
        never = np.where(sc[:L] < sk - eps)[0]
        sset = set(sel.tolist())
        missing = [j for j in must.tolist() if j not in sset]
        assert not missing, (row, "missing above band", missing[:5])
        bad = [j for j in never.tolist() if j in sset]
        assert not bad, (row, "selected below band", bad[:5])
        same = np.array_equal(np.sort(or_idx[r][or_idx[r] >= 0]), sel)
        if gpu_scores is not None and m < L:
            err = np.max(np.abs(gpu_scores[r][:L].astype(np.float64) - sc[:L]))
            stats["max_score_err"] = max(stats["max_score_err"], float(err))
            srt = np.sort(sc[:L])[::-1]
            delta = srt[m - 1] - srt[m]
            if delta > 2 * err:
                assert same, (row, "margin exceeds twice the score error but sets differ", delta, err)
        stats["exact_rows" if same else "band_rows"] += 1
        if tie_groups is not None:
            for grp in tie_groups.get(b, []):
                grp = [j for j in grp if j < L]
                chosen = [j for j in grp if j in sset]
                assert chosen == sorted(grp)[: len(chosen)], (row, "tie group not resolved to lowest positions")
    return stats


def tie_groups_of(k_idx_b, L):
    """Groups (len >= 2) of positions < L whose index-key rows are byte-identical."""
    rows = np.ascontiguousarray(k_idx_b[:L]).view(np.uint8).reshape(L, -1)
    _, inv, cnt = np.unique(rows, axis=0, return_inverse=True, return_counts=True)
    groups = []
    for gid in np.where(cnt > 1)[0]:
        groups.append(sorted(np.where(inv.ravel() == gid)[0].tolist()))
    return groups
