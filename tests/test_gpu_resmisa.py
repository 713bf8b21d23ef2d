"""GPU parity of the selection with a shared linear term and residual heads ("PaperTrace
2.2 · Fine-grained indexing", §2.2, the ResMiSA paragraph): ReLU(z) = z + ReLU(-z) turns
every head's linear part into one dot product with the weighted sum of the head queries,
and only the routed heads keep their non-linear part.

The entry point returns the routed heads; they must be a top-g of the oracle's routing
scores (as for the plain active-head selection) and the tokens a top-k of the oracle's
ResMiSA scores over those heads.  Score tolerance per row (derived from the arithmetic):
the shared query is a sequential fp32 sum over Hidx heads (Hidx rounding steps), its three
bf16 parts hold it to 2^-24 relative, and the scored heads' dot products accumulate d_idx
products in fp32 and Hs slot terms (Hs = 16, 32 or 64 scored slots), so
    |r_gpu - r| <= (2 d_idx + Hidx + Hs + 8) 2^-24 sum_d |k_d| sum_h |w_h q_hd|;
a selected token's score may sit below an unselected one by at most twice that."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from token_selector_gather_amd.inputs import device_workload

pytestmark = pytest.mark.gpu
E4M3 = sa_synth.E4M3


def _say(x):
    print(x, flush=True)


def scored_heads(g):
    return 16 if g + 6 <= 16 else (32 if g + 6 <= 32 else 64)


def gpu_resmisa(W, blk, g):
    P, d = device_workload(W, with_main=False)
    kbar = torch.full((W["B"], W["n_kv"] // blk, W["d_idx"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    sa.sa_block_means(P, d["k_idx"], blk, kbar)
    ws = sa.resmisa_workspace(P, blk, g)
    idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    heads = torch.full((W["B"], W["n_q"], g), -7, dtype=torch.int32, device="cuda")
    sa.sa_resmisa_select(P, d["q_idx"], d["k_idx"], d["w"], kbar, blk, g, idx, ws, heads=heads)
    st = sa.sa_device_status(ws)
    return (kbar.view(torch.int16).cpu().numpy().view(np.uint16), idx.cpu().numpy().reshape(-1, W["k"]),
            heads.cpu().numpy().reshape(-1, g), st)


def resmisa_tolerance(W, rows, g):
    q = gc.decode_f64(W["q_idx"])
    k = gc.decode_f64(W["k_idx"])
    w = np.abs(W["w"].astype(np.float64))
    n = 2 * W["d_idx"] + W["Hidx"] + scored_heads(g) + 8
    out = np.empty((len(rows), W["n_kv"]))
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        u = (w[b, i][:, None] * np.abs(q[b, i])).sum(0)
        out[r] = n * 2.0 ** -24 * (np.abs(k[b]) @ u)
    return out


def check_tokens(W, rows, got_idx, sc, tol):
    """Each row's tokens are a valid top-k of the fp64 scores `sc` up to 2 tol; returns the
    fraction of rows identical to the exact top-k."""
    ref, *_ = orc.select(W, sc, rows)
    same = 0
    for r, row in enumerate(rows):
        s = sc[r]
        L = int(np.isfinite(s).sum())
        gi = got_idx[row]
        n = min(W["k"], L)
        assert (gi[:n] >= 0).all() and (gi[n:] == -1).all() and (np.diff(gi[:n]) > 0).all() and (gi[:n] < L).all(), row
        if n < L:
            sel = np.zeros(L, bool)
            sel[gi[:n]] = True
            assert s[:L][sel].min() >= s[:L][~sel].max() - 2 * tol[r].max(), row
        same += np.array_equal(gi, ref[r])
    return same / len(rows)


def check_rows(W, blk, g, rows, got_idx, got_heads, kbar):
    H = W["Hidx"]
    ref = orc.resmisa_select(W, blk, g, rows, kbar=kbar)
    tr = gc.route_tolerance(W, kbar, rows)
    for r, row in enumerate(rows):
        h = got_heads[row]
        assert (np.diff(h) > 0).all() and h.min() >= 0 and h.max() < H, row
        if g < H:
            dropped = np.setdiff1d(np.arange(H), h)
            assert ref["route"][r, h].min() >= ref["route"][r, dropped].max() - 2 * tr[r], row
    # token stage on the GPU's heads
    sc = orc.resmisa_scores(W, got_heads[rows], rows)
    return check_tokens(W, rows, got_idx, sc, resmisa_tolerance(W, rows, g))


CASES = {
    # 64 heads x 128 e4m3 keys, 10 residual heads: 16 scored slots (the shared query's six
    # parts and the ten negated heads)
    "prefill_h64_e4m3_g10": (dict(B=1, n_q=600, n_kv=600, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=48), 64, 10),
    # 32 residual heads of 64: 38 slots, padded to 64
    "prefill_h64_e4m3_g32": (dict(B=1, n_q=600, n_kv=600, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=48), 64, 32),
    "prefill_h32_bf16_b2_g8": (dict(B=2, n_q=300, n_kv=400, Hidx=32, d_idx=64, k=32, lens=[400, 310]), 32, 8),
    "decode_h64_b5_g16": (dict(B=5, n_q=1, n_kv=5000, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=256,
                               lens=[5000, 3000, 130, 64, 20], q_pos0=[4999, 2999, 129, 63, 19]), 64, 16),
    "noncausal_h16_g4": (dict(B=2, n_q=9, n_kv=700, Hidx=16, d_idx=64, k=40, causal=0, lens=[700, 333]), 16, 4),
    # a shape the streaming score + select takes (64 x 128 e4m3, 4096 rows; 16 scored slots)
    "streaming_h64_e4m3_g10": (dict(B=1, n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=256), 128, 10),
}


def _custom(kw, seed):
    kw = dict(kw)
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    return sa_synth.custom(seed=seed, lens=lens, q_pos0=q_pos0, with_main=False, **kw)


@pytest.mark.parametrize("case", list(CASES))
def test_resmisa_matches_oracle(case):
    kw, blk, g = CASES[case]
    W = _custom(kw, seed=33)
    _say("resmisa %s blk %d g %d" % (case, blk, g))
    kbar, idx, heads, st = gpu_resmisa(W, blk, g)
    assert st == sa.SA_OK
    R = W["B"] * W["n_q"]
    rows = np.arange(R, dtype=np.int32) if R <= 1200 else gc.sample_rows(W, n_each=16, n_rand=48)
    frac = check_rows(W, blk, g, rows, idx, heads, kbar)
    _say("resmisa %s: %.1f%% of rows identical to the oracle" % (case, 100 * frac))


@pytest.mark.parametrize("H,g", [(16, 16), (32, 32)])
def test_resmisa_with_every_head_residual_is_the_flat_selection(H, g):
    # with every head residual the score is the indexer's own (z + ReLU(-z) = ReLU(z) per
    # head): the selection is a top-k of the oracle's flat scores within the tolerance
    W = _custom(dict(B=2, n_q=260, n_kv=700, Hidx=H, d_idx=64, k=40, lens=[700, 450]), seed=35)
    kbar, idx, heads, st = gpu_resmisa(W, 32, g)
    assert st == sa.SA_OK
    assert (heads == np.arange(H)).all()
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    frac = check_tokens(W, rows, idx, orc.scores(W, rows), resmisa_tolerance(W, rows, g))
    _say("resmisa all heads H=%d: %.1f%% of rows identical to the flat oracle" % (H, 100 * frac))


def test_resmisa_rejects_too_many_residual_heads():
    W = _custom(dict(B=1, n_q=64, n_kv=256, Hidx=64, d_idx=64, k=16), seed=37)
    P, d = device_workload(W, with_main=False)
    assert sa.sa_resmisa_workspace_bytes(P, 64, 58) > 0
    assert sa.sa_resmisa_workspace_bytes(P, 64, 59) == 0
    kbar = torch.empty((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((1, 64, 16), dtype=torch.int32, device="cuda")
    ws = sa.resmisa_workspace(P, 64, 58)
    with pytest.raises(RuntimeError):
        sa.sa_resmisa_select(P, d["q_idx"], d["k_idx"], d["w"], kbar, 64, 59, idx, ws)


@pytest.mark.parametrize("cid,blk,g,nrows", [(2, 128, 10, 8), (3, 64, 10, 6)])
def test_resmisa_full_size_sampled_rows(cid, blk, g, nrows):
    W = gc.workload(("misa", cid), cid=cid, with_main=False)
    _say("resmisa full c%d blk %d g %d" % (cid, blk, g))
    kbar, idx, heads, st = gpu_resmisa(W, blk, g)
    assert st == sa.SA_OK
    rng = np.random.default_rng(cid + 100)
    R = W["B"] * W["n_q"]
    rows = np.unique(np.concatenate([rng.choice(R, size=nrows, replace=False), [R - 1]])).astype(np.int32)
    frac = check_rows(W, blk, g, rows, idx, heads, kbar)
    flat, *_ = orc.select(W, orc.scores(W, rows), rows)
    iou = [len(set(a[a >= 0]) & set(f[f >= 0])) / max(1, len(set(a[a >= 0]) | set(f[f >= 0])))
           for a, f in zip(idx[rows], flat)]
    _say("resmisa full c%d: %.0f%% identical to the oracle, IoU with the flat selection %.3f" %
         (cid, 100 * frac, float(np.mean(iou))))
