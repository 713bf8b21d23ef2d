"""Exact-tie groups at the selection cutoff of the planted-needle decode workload.

The generator plants the needles (keys along each query's head-weighted index direction)
but placing a tie group *at the cutoff* needs the score itself, so it is done here with
the oracle (test infrastructure).  For every query row, in order: take the visible
positions sorted by (oracle score desc, position asc); the key at rank k-4 (0-based) is
copied over the keys at ranks k-3 .. k+2, giving seven byte-identical index keys whose
common score straddles the cutoff (four of them fit inside the budget).  The lower-position
tie rule ("PaperTrace 2.2 · Fine-grained indexing", §2.1 and §3.1) then decides exactly
which four are selected.  Positions already used by an earlier group or a needle are left
alone.
"""
import numpy as np

from oracle import oracle as orc


def plant_cutoff_ties(W, span=(-4, 3)):
    W = dict(W)
    W["k_idx"] = W["k_idx"].copy()
    k = W["k"]
    used = set(int(x) for x in np.asarray(W.get("needle_pos", np.zeros(0))).reshape(-1))
    groups = {}
    for row in range(W["B"] * W["n_q"]):
        b, i = divmod(row, W["n_q"])
        sc = orc.scores(W, np.array([row], np.int32))[0]
        vis = np.where(np.isfinite(sc))[0]
        order = vis[np.lexsort((vis, -sc[vis]))]
        ranks = list(range(k + span[0], k + span[1]))
        members = [int(order[r]) for r in ranks if 0 <= r < order.size]
        if any(m in used for m in members) or len(members) < 2:
            continue
        src = members[0]
        for m in members[1:]:
            W["k_idx"][b, m] = W["k_idx"][b, src]
        used.update(members)
        groups[row] = sorted(members)
    W["tie_groups_planted"] = groups
    return W
