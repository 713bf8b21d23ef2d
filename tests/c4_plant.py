"""Exact-tie groups at the selection cutoff of the planted-needle decode workload.

The generator plants the needles (keys along each query's head-weighted index direction)
but placing a tie group *at the cutoff* needs the score itself, so it is done here with
the oracle (test infrastructure).  For every query row: take the visible positions
sorted by (oracle score desc, position asc); starting at rank k-4 (0-based), the first
seven positions not used by a needle or another group form the group, and the key of the
first is copied over the other six.  The seven byte-identical index keys share the score of
rank k-4, so exactly four of them fit inside the budget, and the lower-position tie rule
("PaperTrace 2.2 · Fine-grained indexing", §2.1 and §3.1) decides which four.  The history
is shared by all query rows, so a group can move another row's cutoff; rows whose group no
longer straddles its cutoff are planted again (a few passes).
"""
import numpy as np

from oracle import oracle as orc


def _straddling(W, groups, rows):
    sc = orc.scores(W, rows)
    idx, *_ = orc.select(W, sc, rows)
    ok = {}
    for r, row in enumerate(rows.tolist()):
        if row in groups:
            chosen = set(idx[r].tolist()) & set(groups[row])
            ok[row] = 0 < len(chosen) < len(groups[row])
    return sc, ok


def plant_cutoff_ties(W, start=-4, size=7, passes=6):
    W = dict(W)
    W["k_idx"] = W["k_idx"].copy()
    k = W["k"]
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    used = set(int(x) for x in np.asarray(W.get("needle_pos", np.zeros(0))).reshape(-1))
    groups = {}
    todo = rows.tolist()
    sc = orc.scores(W, rows)
    for _ in range(passes):
        for row in todo:
            b = row // W["n_q"]
            s = sc[row]
            vis = np.where(np.isfinite(s))[0]
            order = vis[np.lexsort((vis, -s[vis]))]
            members = [int(j) for j in order[max(0, k + start):] if int(j) not in used][:size]
            if len(members) < 2:
                continue
            for m in members[1:]:
                W["k_idx"][b, m] = W["k_idx"][b, members[0]]
            used.update(members)
            groups[row] = sorted(members)
        sc, ok = _straddling(W, groups, rows)
        todo = [row for row in rows.tolist() if not ok.get(row, False)]
        if not todo:
            break
    W["tie_groups_planted"] = {row: grp for row, grp in groups.items() if ok.get(row, False)}
    return W
