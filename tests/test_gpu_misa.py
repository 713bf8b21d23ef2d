"""GPU parity of the active-head selection ("PaperTrace 2.2 · Fine-grained indexing", the
MISA paragraphs): routing scores over the block representatives, the g best heads per
query row, token scores over those heads and the top-k, against the oracle.

As for the hierarchical selection, the head choice and the token choice are integer
decisions on fp32 (GPU) versus fp64 (oracle) scores: each row's heads (returned by the
entry point) must be a top-g of the oracle's routing scores and its tokens a top-k of the
oracle's scores over those heads, both up to twice the score tolerance (exactly the
oracle's choice where the cutoff is separated by more).  Both sides use the GPU's bf16
block representatives, which are checked against the oracle's separately."""
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


def gpu_misa(W, blk, g):
    P, d = device_workload(W, with_main=False)
    kbar = torch.full((W["B"], W["n_kv"] // blk, W["d_idx"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    sa.sa_block_means(P, d["k_idx"], blk, kbar)
    ws = sa.misa_workspace(P, blk, g)
    idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    heads = torch.full((W["B"], W["n_q"], g), -7, dtype=torch.int32, device="cuda")
    sa.sa_misa_select(P, d["q_idx"], d["k_idx"], d["w"], kbar, blk, g, idx, ws, heads=heads)
    st = sa.sa_device_status(ws)
    return (kbar.view(torch.int16).cpu().numpy().view(np.uint16), idx.cpu().numpy().reshape(-1, W["k"]),
            heads.cpu().numpy().reshape(-1, g), st)


def check_rows(W, blk, g, rows, got_idx, got_heads, kbar):
    ref = orc.misa_select(W, blk, g, rows, kbar=kbar)
    tr = gc.route_tolerance(W, kbar, rows)
    H = W["Hidx"]
    for r, row in enumerate(rows):
        h = got_heads[row]
        assert (np.diff(h) > 0).all() and h.min() >= 0 and h.max() < H, row
        if g < H:
            dropped = np.setdiff1d(np.arange(H), h)
            assert ref["route"][r, h].min() >= ref["route"][r, dropped].max() - 2 * tr[r], row
    # token stage on the GPU's heads
    tok = orc.misa_select(W, blk, g, rows, kbar=kbar, heads=got_heads[rows])
    tt = gc.score_tolerance(W, rows)  # all heads: an upper bound for any subset
    same = 0
    for r, row in enumerate(rows):
        sc = tok["scores"][r]
        L = int(np.isfinite(sc).sum())
        gi = got_idx[row]
        n = min(W["k"], L)
        assert (gi[:n] >= 0).all() and (gi[n:] == -1).all() and (np.diff(gi[:n]) > 0).all() and (gi[:n] < L).all(), row
        if n < L:
            sel = np.zeros(L, bool)
            sel[gi[:n]] = True
            assert sc[:L][sel].min() >= sc[:L][~sel].max() - 2 * tt[r].max(), row
        same += np.array_equal(got_heads[row], ref["heads"][r]) and np.array_equal(gi, ref["idx"][r])
    return same / len(rows)


CASES = {
    "prefill_h64_e4m3": (dict(B=1, n_q=600, n_kv=600, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=48), 64, 16),
    "prefill_h32_bf16_b2": (dict(B=2, n_q=300, n_kv=400, Hidx=32, d_idx=64, k=32, lens=[400, 310]), 32, 8),
    "decode_h64_b5": (dict(B=5, n_q=1, n_kv=5000, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=256,
                           lens=[5000, 3000, 130, 64, 20], q_pos0=[4999, 2999, 129, 63, 19]), 64, 16),
    "noncausal_h16": (dict(B=2, n_q=9, n_kv=700, Hidx=16, d_idx=64, k=40, causal=0, lens=[700, 333]), 16, 4),
}


@pytest.mark.parametrize("case", list(CASES))
def test_misa_matches_oracle(case):
    kw, blk, g = CASES[case]
    kw = dict(kw)
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    W = sa_synth.custom(seed=31, lens=lens, q_pos0=q_pos0, with_main=False, **kw)
    _say("misa %s blk %d g %d" % (case, blk, g))
    kbar, idx, heads, st = gpu_misa(W, blk, g)
    assert st == sa.SA_OK
    # the representatives the routing used against the oracle's own
    ref_kbar = orc.block_means(W, blk)
    if W["kidx_dtype"] == E4M3:  # fp32 sums of e4m3 keys are exact: identical representatives
        np.testing.assert_array_equal(kbar, ref_kbar)
    else:  # fp32 sums of bf16 keys: at most one bf16 unit apart after the rounding
        assert np.abs(kbar.astype(np.int64) - ref_kbar.astype(np.int64)).max() <= 1
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    frac = check_rows(W, blk, g, rows, idx, heads, kbar)
    _say("misa %s: %.1f%% of rows identical to the oracle" % (case, 100 * frac))


def test_misa_with_every_head_is_the_gpu_flat_selection():
    # all heads active, in ascending order: the same queries, weights and kernels as the
    # flat score, so the selection is the flat one bit for bit
    W = sa_synth.custom(seed=6, B=1, n_q=520, n_kv=520, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=32, with_main=False)
    _, idx, heads, st = gpu_misa(W, 64, 64)
    assert st == sa.SA_OK
    assert (heads == np.arange(64)).all()
    flat, _, st2 = gc.gpu_topk(W, gc.gpu_scores(W))
    assert st2 == sa.SA_OK
    np.testing.assert_array_equal(idx, flat.reshape(idx.shape))


@pytest.mark.parametrize("cid,blk,g,nrows", [(2, 128, 16, 10), (3, 64, 16, 6)])
def test_misa_full_size_sampled_rows(cid, blk, g, nrows):
    W = gc.workload(("misa", cid), cid=cid, with_main=False)
    _say("misa full c%d blk %d g %d" % (cid, blk, g))
    kbar, idx, heads, st = gpu_misa(W, blk, g)
    assert st == sa.SA_OK
    rng = np.random.default_rng(cid)
    R = W["B"] * W["n_q"]
    rows = np.unique(np.concatenate([rng.choice(R, size=nrows, replace=False), [R - 1]])).astype(np.int32)
    bs = np.unique(rows // W["n_q"])
    np.testing.assert_array_equal(kbar[bs], orc.block_means(W, blk, batches=bs))
    frac = check_rows(W, blk, g, rows, idx, heads, kbar)
    flat, *_ = orc.select(W, orc.scores(W, rows), rows)
    iou = [len(set(a[a >= 0]) & set(f[f >= 0])) / max(1, len(set(a[a >= 0]) | set(f[f >= 0])))
           for a, f in zip(idx[rows], flat)]
    _say("misa full c%d: %.0f%% identical to the oracle, IoU with the flat selection %.3f" % (cid, 100 * frac,
                                                                                          float(np.mean(iou))))
