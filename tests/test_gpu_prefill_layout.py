"""GPU parity of the indexer's many-row prefill layout (one pass over the history per block
of query rows, keys widened to bf16 once per chunk), which serves workloads with thousands
of query rows.  Sampled rows of the standalone score call (invisible entries filled; NaN
for the rows and keys with non-finite index inputs) and of the fused call (finite inputs,
plain ReLU) against the oracle ("PaperTrace 2.2 · Fine-grained indexing", §2.1 eq. (1);
the score definition of the Lightning indexer)."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu
BF16, E4M3 = sa_synth.BF16, sa_synth.E4M3

MAIN = dict(Hq=2, Hkv=2, d_qk=64, d_v=64)
CASES = {
    # latent-prefill index dimensions (64 heads x 128, e4m3 keys), 1024 blocks of 8 rows
    "h64_d128_e4m3_n8192": dict(n_q=8192, n_kv=8192, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=256, **MAIN),
    # 32 heads x 64, bf16 keys, four batches with padding (one nearly empty)
    "h32_d64_bf16_b4_n4096": dict(B=4, n_q=4096, n_kv=4096, Hidx=32, d_idx=64, kidx_dtype=BF16, k=128,
                                  lens=[4096, 3001, 4096, 17], **MAIN),
    # 16 heads x 64, e4m3 keys, chunked prefill (queries start late in the history)
    "h16_d64_e4m3_b8_n2048": dict(B=8, n_q=2048, n_kv=2500, Hidx=16, d_idx=64, kidx_dtype=E4M3, k=64,
                                  q_pos0=[452] * 8, lens=[2500] * 8, **MAIN),
}


def _say(x):
    print(x, flush=True)


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_layout_scores_and_selection(case):
    kw = dict(CASES[case])
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    W = sa_synth.custom(seed=7, lens=lens, q_pos0=q_pos0, **kw)
    rows = gc.sample_rows(W, n_each=8, n_rand=48)
    _say("prefill layout %s: %d rows" % (case, rows.size))
    sc = gc.gpu_scores(W).reshape(-1, W["n_kv"])[rows].cpu().numpy()
    ref = orc.scores(W, rows)
    inv = np.isneginf(ref)
    assert np.isneginf(sc[inv]).all(), "invisible entries must be -inf"
    tol = gc.score_tolerance(W, rows)
    err = np.abs(sc[~inv].astype(np.float64) - ref[~inv])
    assert (err <= tol[~inv]).all(), float((err - tol[~inv]).max())
    r = gc.full_check(W, rows=rows, check_sparse=False)
    _say("prefill layout %s: exact rows %d band rows %d" % (case, r["exact_rows"], r["band_rows"]))


# non-finite index inputs in the standalone score call: a query row with a bad element scores
# NaN on every visible key, a bad key scores NaN in every row that sees it, every other
# visible entry is the clean workload's score, and the selection reports the condition
NONFINITE = {
    # e4m3 keys: a negative NaN query element, +inf and -inf query elements, two NaN keys
    "h64_d128_e4m3": dict(kw=dict(B=1, n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=64),
                          q=[(700, 5, 17, 0xFFC0), (2900, 63, 127, 0x7F80), (4095, 0, 0, 0xFF80)],
                          kk=[(300, 9, 0x7F), (3999, 127, 0xFF)]),
    # bf16 keys: a -inf key and a NaN key; a positive NaN query element
    "h32_d64_bf16": dict(kw=dict(B=4, n_q=2048, n_kv=2048, Hidx=32, d_idx=64, kidx_dtype=BF16, k=64),
                         q=[(1500, 31, 2, 0x7FC0)], kk=[(0, 63, 0xFF80), (1024, 0, 0xFFC0)]),
}


@pytest.mark.parametrize("case", list(NONFINITE))
def test_prefill_layout_standalone_scores_keep_nonfinite_inputs_visible(case):
    spec = NONFINITE[case]
    W = sa_synth.custom(seed=11, **spec["kw"], **MAIN)
    Wb = W.__class__(W)
    Wb["q_idx"], Wb["k_idx"] = W["q_idx"].copy(), W["k_idx"].copy()
    bad_rows, bad_keys = [], []
    for n, (i, h, d, code) in enumerate(spec["q"]):
        b = n % W["B"]
        Wb["q_idx"][b, i, h, d] = code
        bad_rows.append((b, i))
    for n, (j, d, code) in enumerate(spec["kk"]):
        b = n % W["B"]
        Wb["k_idx"][b, j, d] = code
        bad_keys.append((b, j))
    _say("standalone non-finite %s: rows %s keys %s" % (case, bad_rows, bad_keys))
    sc = gc.gpu_scores(Wb).cpu().numpy()
    n_q, n_kv = W["n_q"], W["n_kv"]
    vis = np.zeros((W["B"], n_q, n_kv), bool)
    for b in range(W["B"]):
        L = np.minimum(np.arange(n_q) + int(W["q_pos0"][b]) + 1, int(W["kv_len"][b]))
        vis[b] = np.arange(n_kv)[None, :] < L[:, None]
    bad = np.zeros_like(vis)
    for b, i in bad_rows:
        bad[b, i] = True
    for b, j in bad_keys:
        bad[b, :, j] = True
    bad &= vis
    assert bad.sum() > 0
    assert np.isnan(sc[bad]).all(), "every visible entry of a bad row or key must be NaN"
    assert np.isneginf(sc[~vis]).all(), "invisible entries must be -inf"
    assert np.isfinite(sc[vis & ~bad]).all()
    # sampled clean rows (and the bad rows' neighbours) match the clean workload's oracle
    rows = gc.sample_rows(W, n_each=4, n_rand=24)
    extra = [b * n_q + min(i + 1, n_q - 1) for b, i in bad_rows]
    rows = np.unique(np.concatenate([rows, np.asarray(extra, rows.dtype)]))
    rows = np.asarray([r for r in rows if (divmod(int(r), n_q)) not in bad_rows], rows.dtype)
    ref = orc.scores(W, rows)
    tol = gc.score_tolerance(W, rows)
    got = sc.reshape(-1, n_kv)[rows]
    ok = vis.reshape(-1, n_kv)[rows] & ~bad.reshape(-1, n_kv)[rows]
    err = np.abs(got[ok].astype(np.float64) - ref[ok])
    assert (err <= tol[ok]).all(), float((err - tol[ok]).max())
    # the selection over these scores reports the non-finite input
    _, _, st = gc.gpu_topk(Wb, torch.from_numpy(sc).cuda())
    assert st == sa.SA_ERR_NONFINITE
