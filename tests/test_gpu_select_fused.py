"""GPU parity of the fused score + select (sa_select, and sa_select_attend's selection):
the streaming top-k that never stores the scores ("PaperTrace 2.2 · Fine-grained
indexing", §2.1: score the history slice by slice, keep local candidates, merge down to k;
the result is the global top-k).  The scores are computed by the same MFMA code as the
standalone score call, so the selection must equal sa_indexer_score followed by sa_topk
bit for bit -- including every exact tie, which goes to the lower position -- and stay
inside the oracle's band.  Small budgets make the candidate lists overflow and be cut back
many times per row; key pools with few distinct keys make most scores tie."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from tests.checker import check_index_rows
from token_selector_gather_amd.inputs import device_workload

pytestmark = pytest.mark.gpu
BF16, E4M3, F32 = sa_synth.BF16, sa_synth.E4M3, sa_synth.F32


def _say(x):
    print(x, flush=True)


def two_pass(W, P, d):
    sc = torch.empty((W["B"], W["n_q"], W["n_kv"]), dtype=torch.float32, device="cuda")
    sa.sa_indexer_score(P, d["q_idx"], d["k_idx"], d["w"], sc)
    ws = sa.workspace(P, sa.SA_OP_TOPK)
    idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    sa.sa_topk(P, sc, W["n_kv"], idx, None, ws)
    assert sa.sa_device_status(ws) == sa.SA_OK
    return idx, sc


def fused(W, P, d):
    ws = sa.workspace(P, sa.SA_OP_SELECT)
    idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    sa.sa_select(P, d["q_idx"], d["k_idx"], d["w"], idx, ws)
    return idx, sa.sa_device_status(ws)


def _first_diff(a, b):
    bad = torch.nonzero((a != b).any(dim=-1).reshape(-1)).reshape(-1)
    return int(bad[0]) if bad.numel() else None


CASES = {
    # 64 heads x 128, e4m3 keys (the latent prefill's indexer), k = 64: lists of 256 entries
    # cut back to 64 about every 200 keys over histories of up to 4096
    "h64_d128_e4m3_k64": dict(n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=64),
    # the same with a budget of 512 and two padded batches
    "h64_d128_e4m3_k512_b2": dict(B=2, n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=512,
                                  lens=[4096, 2500]),
    # 64 heads x 64, bf16 keys, non-causal: every row sees the same 3000 keys
    "h64_d64_bf16_noncausal": dict(B=1, n_q=4096, n_kv=3000, Hidx=64, d_idx=64, kidx_dtype=BF16, k=200,
                                   causal=0),
    # 32 heads x 64 (16 rows per block), chunked prefill (queries start late in the history)
    "h32_d64_e4m3_chunked": dict(B=2, n_q=4096, n_kv=6000, Hidx=32, d_idx=64, kidx_dtype=E4M3, k=128,
                                 q_pos0=[1904, 1000], lens=[6000, 5096]),
    # 16 heads x 128 (32 rows per block, two lane-group queries per lane), ragged padding
    "h16_d128_bf16": dict(B=4, n_q=4096, n_kv=2048, Hidx=16, d_idx=128, kidx_dtype=BF16, k=96,
                          lens=[2048, 1500, 2048, 33]),
    # a budget above a fifth of the histories: rows shorter than k return their whole prefix
    "h64_d128_e4m3_k900": dict(n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=900),
}


def _workload(kw, seed=41, with_main=False):
    kw = dict(kw)
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    main = dict(Hq=2, Hkv=2, d_qk=64, d_v=64)
    return sa_synth.custom(seed=seed, lens=lens, q_pos0=q_pos0, with_main=with_main, **main, **kw)


@pytest.mark.parametrize("case", list(CASES))
def test_fused_selection_equals_two_pass(case):
    W = _workload(CASES[case])
    P, d = device_workload(W, with_main=False)
    _say("fused select %s" % case)
    ref, sc = two_pass(W, P, d)
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    r = _first_diff(got, ref)
    assert r is None, ("row", r, got.reshape(-1, W["k"])[r][:16].tolist(), ref.reshape(-1, W["k"])[r][:16].tolist())
    # the oracle's band on sampled rows
    rows = gc.sample_rows(W, n_each=6, n_rand=20)
    ref_sc = orc.scores(W, rows)
    ref_idx, sk, _, _ = orc.select(W, ref_sc, rows)
    g = got.reshape(-1, W["k"]).cpu().numpy()[rows]
    gsc = sc.reshape(-1, W["n_kv"]).cpu().numpy()[rows]
    s = check_index_rows(W, rows, g, ref_sc, ref_idx, sk, gpu_scores=gsc)
    _say("fused select %s: equal to two-pass; oracle exact rows %d band rows %d" % (case, s["exact_rows"],
                                                                                  s["band_rows"]))


@pytest.mark.parametrize("pool", [1, 3, 17])
def test_fused_selection_with_heavy_exact_ties(pool):
    # index keys drawn from `pool` distinct rows: scores tie in large groups, and the lists
    # are cut back inside tie groups; ties must go to the lowest positions as in the
    # two-pass selection
    W = _workload(dict(n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=100), seed=43)
    rng = np.random.default_rng(pool)
    pick = rng.integers(0, pool, W["n_kv"])
    W["k_idx"] = np.ascontiguousarray(W["k_idx"][:, pick, :])
    P, d = device_workload(W, with_main=False)
    _say("fused select ties pool=%d" % pool)
    ref, _ = two_pass(W, P, d)
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    r = _first_diff(got, ref)
    assert r is None, ("row", r)
    if pool == 1:  # every score equal: the first k visible positions
        g = got.reshape(-1, W["k"]).cpu().numpy()
        for i in (0, 99, 100, 2000, 4095):
            m = min(W["k"], i + 1)
            assert g[i, :m].tolist() == list(range(m)) and (g[i, m:] == -1).all()


@pytest.mark.parametrize("sign", ["alternating", "negative", "sparse"])
@pytest.mark.parametrize("case", ["h64_d128_e4m3_k64", "h16_d128_bf16", "h32_d64_e4m3_chunked"])
def test_fused_selection_with_signed_scores(case, sign):
    # head weights of both signs (scores straddle zero), all negative (every score <= 0), or
    # zero on all but three heads (about 1/8 of the scores are exactly zero): the histogram
    # bins, uniform in score, must stay exact across the sign change and the zero ties
    W = _workload(CASES[case], seed=51)
    w = W["w"].astype(np.float32)
    H = W["Hidx"]
    if sign == "alternating":
        w = w * np.where(np.arange(H) % 2 == 0, 1.0, -1.0).astype(np.float32)
    elif sign == "negative":
        w = -w
    else:
        w = w * (np.arange(H) < 3).astype(np.float32)
    W["w"] = np.ascontiguousarray(w)
    P, d = device_workload(W, with_main=False)
    _say("fused select %s, %s weights" % (case, sign))
    ref, sc = two_pass(W, P, d)
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    r = _first_diff(got, ref)
    assert r is None, ("row", r)
    rows = gc.sample_rows(W, n_each=4, n_rand=12)
    ref_sc = orc.scores(W, rows)
    ref_idx, sk, _, _ = orc.select(W, ref_sc, rows)
    g = got.reshape(-1, W["k"]).cpu().numpy()[rows]
    gsc = sc.reshape(-1, W["n_kv"]).cpu().numpy()[rows]
    check_index_rows(W, rows, g, ref_sc, ref_idx, sk, gpu_scores=gsc)


def test_fused_selection_with_empty_and_tiny_histories():
    # a batch whose history is empty (every row padded), one of 37 positions (rows shorter
    # than k return their whole prefix) and a chunked one whose first rows sit at position 0
    W = _workload(dict(B=4, n_q=1024, n_kv=3000, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=64,
                       lens=[3000, 0, 37, 2000], q_pos0=[1976, 0, 0, 0]), seed=53)
    P, d = device_workload(W, with_main=False)
    ref, _ = two_pass(W, P, d)
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    assert _first_diff(got, ref) is None
    g = got.cpu().numpy()
    assert (g[1] == -1).all()                            # empty history: nothing selected
    assert (g[2, 37:] == -1).all()                       # padded rows of the 37-position batch
    for i in (0, 5, 36):                                 # rows shorter than k: the whole prefix
        assert g[2, i, : i + 1].tolist() == list(range(i + 1)) and (g[2, i, i + 1:] == -1).all()
    assert g[3, 0, 0] == 0 and (g[3, 0, 1:] == -1).all()  # a row at position 0 sees only itself


def test_select_attend_uses_the_fused_selection():
    # the fused call's selection (idx_out) equals sa_select's and the attention matches the
    # oracle on sampled rows
    W = _workload(dict(n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=128), seed=45, with_main=True)
    P, d = device_workload(W)
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    idx, O, lse, st2 = gc.gpu_select_attend(W)
    assert st2 == sa.SA_OK
    assert np.array_equal(idx, got.cpu().numpy())
    rows = gc.sample_rows(W, n_each=4, n_rand=12)
    O_or, lse_or = orc.attend(W, idx.reshape(-1, W["k"])[rows], rows)
    gc.compare_attention(W, rows, O, lse, O_or, lse_or)


def test_fused_shape_with_f32_index_inputs_selects_in_row_slices():
    # a shape the streaming form takes, but with f32 index queries: the call scores and
    # selects slices of rows through the same workspace, with the two-pass result
    W = _workload(dict(n_q=4096, n_kv=2048, Hidx=64, d_idx=64, qidx_dtype=F32, kidx_dtype=BF16, k=64), seed=47)
    P, d = device_workload(W, with_main=False)
    ref, _ = two_pass(W, P, d)
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    assert _first_diff(got, ref) is None


@pytest.mark.parametrize("where", ["query", "weight", "key", "padded_query"])
def test_fused_selection_reports_nonfinite_inputs(where):
    W = _workload(dict(B=2, n_q=4096, n_kv=4096, Hidx=64, d_idx=128, kidx_dtype=E4M3, k=64, lens=[4096, 3000]),
                  seed=49)
    P, d = device_workload(W, with_main=False)
    if where == "query":
        d["q_idx"][0, 1234, 17, 5] = float("nan")
    elif where == "weight":
        d["w"][1, 2000, 3] = float("inf")
    elif where == "key":
        d["k_idx"].view(torch.uint8)[1, 2999, 100] = 0xFF  # e4m3 NaN, visible to batch 1's late rows
    else:  # a padded row of batch 1 (q_pos >= kv_len) is not valid: its inputs are not checked
        d["q_idx"][1, 3500, 0, 0] = float("nan")
    _, st = fused(W, P, d)
    assert st == (sa.SA_OK if where == "padded_query" else sa.SA_ERR_NONFINITE), where


def test_fused_selection_full_size_latent_prefill():
    # the latent prefill at full size (n = 32768, 64 x 128 e4m3 index, k = 2048): the fused
    # selection equals the two-pass one on every row
    _say("fused select full c2: generate")
    W = gc.workload(("sel", 2), cid=2, with_main=False)
    P, d = device_workload(W, with_main=False)
    _say("fused select full c2: two-pass")
    ref, sc = two_pass(W, P, d)
    del sc
    torch.cuda.empty_cache()
    _say("fused select full c2: fused")
    got, st = fused(W, P, d)
    assert st == sa.SA_OK
    r = _first_diff(got, ref)
    assert r is None, ("row", r)
    _say("fused select full c2: all %d rows equal" % (W["B"] * W["n_q"]))
