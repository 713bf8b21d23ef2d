"""GPU parity of the hierarchical selection ("PaperTrace 2.2 · Fine-grained indexing", the
HISA paragraphs): block representatives, block top-k_b, token top-k inside the kept blocks
and the open block, against the oracle on the same bytes.

The block and token selections are integer decisions taken on fp32 scores (GPU) and fp64
scores (oracle).  Each row's kept blocks (returned by the entry point) must be a top-k_b of
its visible complete blocks and its tokens a top-k of the candidates those blocks give,
both up to twice the score tolerance: where the cutoff is separated by more than that, the
choice is the oracle's exactly; inside the band any order is valid.  The representatives
are compared separately, and the oracle's stages take the GPU's representatives, so both
sides decide on the same bf16 block keys."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from token_selector_gather_amd.inputs import device_workload

pytestmark = pytest.mark.gpu
BF16, E4M3 = sa_synth.BF16, sa_synth.E4M3


def _say(x):
    print(x, flush=True)


def gpu_hisa(W, blk, kb):
    P, d = device_workload(W, with_main=False)
    nb = W["n_kv"] // blk
    kbar = torch.full((W["B"], nb, W["d_idx"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    sa.sa_block_means(P, d["k_idx"], blk, kbar)
    ws = sa.hisa_workspace(P, blk, kb)
    idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    blocks = torch.full((W["B"], W["n_q"], kb), -7, dtype=torch.int32, device="cuda")
    sa.sa_hisa_select(P, d["q_idx"], d["k_idx"], d["w"], kbar, blk, kb, idx, ws, blocks=blocks)
    st = sa.sa_device_status(ws)
    kb_np = kbar.view(torch.int16).cpu().numpy().view(np.uint16)
    return kb_np, idx.cpu().numpy().reshape(-1, W["k"]), blocks.cpu().numpy().reshape(-1, kb), st


def block_tolerance(W, kbar, rows):
    """Bound on |block score (GPU) - block score (oracle)| per row, as for token scores."""
    q = gc.decode_f64(W["q_idx"])
    kb = orc.decode_array(kbar)
    w = np.abs(W["w"].astype(np.float64))
    n = W["d_idx"] + W["Hidx"] + 2
    out = np.empty(len(rows))
    for r, row in enumerate(rows):
        b, i = divmod(int(row), W["n_q"])
        u = (w[b, i][:, None] * np.abs(q[b, i])).sum(0)
        out[r] = 2 * n * 2.0 ** -24 * (np.abs(kb[b]) @ u).max()
    return out


def check_rows(W, blk, kb, rows, got_idx, got_blocks, kbar):
    """Validity of every listed row within tolerance; returns the fraction equal to the oracle."""
    ref = orc.hisa_select(W, blk, kb, rows, kbar=kbar)
    tb = block_tolerance(W, kbar, rows)
    tt = gc.score_tolerance(W, rows)
    bsc, tsc = ref["block_scores"], ref["token_scores"]
    L = np.isfinite(tsc).sum(axis=1)
    K = W["k"]
    same = 0
    for r, row in enumerate(rows):
        P = int(L[r]) // blk
        nb = min(kb, P)
        g = got_blocks[row]
        # kept blocks: nb visible complete blocks, ascending, none beaten by a dropped block
        assert (g[:nb] >= 0).all() and (g[:nb] < P).all() and (np.diff(g[:nb]) > 0).all() and (g[nb:] == -1).all(), row
        if nb < P:
            dropped = np.setdiff1d(np.arange(P), g[:nb])
            assert bsc[r, g[:nb]].min() >= bsc[r, dropped].max() - 2 * tb[r], row
        # tokens: a top-k of the candidates of those blocks plus the open block
        cand = np.concatenate([np.arange(B * blk, (B + 1) * blk) for B in g[:nb]] + [np.arange(P * blk, L[r])])
        gi = got_idx[row]
        n = min(K, cand.size)
        assert (gi[n:] == -1).all() and (np.diff(gi[:n]) > 0).all() and np.isin(gi[:n], cand).all(), row
        if n < cand.size:
            sel = np.isin(cand, gi[:n])
            assert tsc[r, cand[sel]].min() >= tsc[r, cand[~sel]].max() - 2 * tt[r, cand].max(), row
        same += np.array_equal(g, ref["blocks"][r]) and np.array_equal(gi, ref["idx"][r])
    return same / len(rows)

CASES = {
    # decode: one row per batch, ragged lengths, e4m3 keys, 64 x 128 index heads
    "decode_b6_e4m3": (dict(B=6, n_q=1, n_kv=6000, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=256, causal=1,
                            lens=[6000, 4100, 777, 64, 63, 5000], q_pos0=[5999, 4099, 776, 63, 62, 4999]), 64, 8),
    # causal prefill, bf16 keys: rows shorter than a block, than k_b blocks, and longer
    "prefill_bf16": (dict(B=2, n_q=300, n_kv=320, Hidx=16, d_idx=64, k=24, lens=[320, 250]), 16, 5),
    # non-causal rows with padding, e4m3 keys, 32 heads
    "noncausal_e4m3": (dict(B=3, n_q=7, n_kv=2048, Hidx=32, d_idx=64, kidx_dtype=E4M3, k=64, causal=0,
                            lens=[2048, 1500, 100]), 32, 6),
}


@pytest.mark.parametrize("case", list(CASES))
def test_hisa_matches_oracle(case):
    kw, blk, kb = CASES[case]
    kw = dict(kw)
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    W = sa_synth.custom(seed=21, lens=lens, q_pos0=q_pos0, with_main=False, **kw)
    _say("hisa %s blk %d kb %d" % (case, blk, kb))
    kbar, idx, blocks, st = gpu_hisa(W, blk, kb)
    assert st == sa.SA_OK
    ref_kbar = orc.block_means(W, blk)
    if W["kidx_dtype"] == E4M3:  # fp32 sums of e4m3 keys are exact: identical representatives
        np.testing.assert_array_equal(kbar, ref_kbar)
    else:
        assert np.abs(kbar.astype(np.int64) - ref_kbar.astype(np.int64)).max() <= 1
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    frac = check_rows(W, blk, kb, rows, idx, blocks, kbar)
    _say("hisa %s: %.1f%% of rows identical to the oracle" % (case, 100 * frac))


def test_hisa_keeping_every_block_is_the_gpu_flat_selection():
    # every block kept: the candidates are the whole visible history, scored by the same
    # decode kernel in the same order, so the selection is the flat one bit for bit
    W = sa_synth.custom(seed=4, B=4, n_q=1, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=128,
                        lens=[4096, 3000, 2049, 130], q_pos0=[4095, 2999, 2048, 129], with_main=False)
    _, idx, _, st = gpu_hisa(W, 64, 4096 // 64)
    assert st == sa.SA_OK
    flat, _, st2 = gc.gpu_topk(W, gc.gpu_scores(W))
    assert st2 == sa.SA_OK
    np.testing.assert_array_equal(idx, flat.reshape(idx.shape))


@pytest.mark.parametrize("cid,blk,kb,nrows", [(3, 64, 64, 6), (4, 64, 32, 8)])
def test_hisa_full_size_sampled_rows(cid, blk, kb, nrows):
    W = gc.workload(("hisa", cid), cid=cid, with_main=False)
    _say("hisa full c%d blk %d kb %d" % (cid, blk, kb))
    kbar, idx, blocks, st = gpu_hisa(W, blk, kb)
    assert st == sa.SA_OK
    rng = np.random.default_rng(cid)
    rows = np.sort(rng.choice(W["B"] * W["n_q"], size=min(nrows, W["B"] * W["n_q"]), replace=False)).astype(np.int32)
    bs = np.unique(rows // W["n_q"])
    np.testing.assert_array_equal(kbar[bs], orc.block_means(W, blk, batches=bs))
    frac = check_rows(W, blk, kb, rows, idx, blocks, kbar)
    # overlap with the flat selection (informational: the synthetic keys carry no block structure)
    flat, *_ = orc.select(W, orc.scores(W, rows), rows)
    iou = [len(set(a[a >= 0]) & set(f[f >= 0])) / max(1, len(set(a[a >= 0]) | set(f[f >= 0])))
           for a, f in zip(idx[rows], flat)]
    _say("hisa full c%d: %.0f%% identical to the oracle, IoU with the flat selection %.3f" % (cid, 100 * frac,
                                                                                          float(np.mean(iou))))
