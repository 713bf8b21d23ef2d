"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it follows.  None of them re-types the oracle's formula:
they use the pages' printed worked examples, hand-worked values, identities stated on
the pages, closed forms, brute force on tiny inputs, and library routines (torch's
scaled_dot_product_attention, numpy's lexsort, torch's float8 / bfloat16 casts).
"""
import math

import numpy as np
import pytest
import torch

import sa_synth
from oracle import oracle as orc
from tests._util import tiny, all_rows, full_idx, rand_f32
from tests.conftest import golden

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ------------------------------------------------------------------ codecs

def test_e4m3_decoder_matches_torch_float8_and_spot_values():
    # OCP e4m3fn: 0x7e = 448 (max finite), 0x38 = 1.0, 0x08 = 2^-6 (min normal), 0x01 = 2^-9.
    spot = {0x7E: 448.0, 0x38: 1.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x00: 0.0, 0xB8: -1.0, 0xFE: -448.0,
            0x40: 2.0, 0x3C: 1.5}
    for code, val in spot.items():
        assert orc.decode(orc.E4M3, code) == val
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for code in range(256):
        got = orc.decode(orc.E4M3, code)
        if code in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(ref[code])
        else:
            assert got == ref[code], hex(code)


def test_bf16_decoder_matches_torch_bfloat16():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits[:4096], ref):
        g = orc.decode(orc.BF16, int(b))
        assert (math.isnan(g) and math.isnan(r)) or g == r
    assert orc.decode(orc.BF16, 0x3F80) == 1.0 and orc.decode(orc.BF16, 0xC000) == -2.0


def test_synth_encoders_round_trip_and_match_torch():
    # every finite e4m3 code survives decode -> encode; RNE fp32 -> e4m3 agrees with torch
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.int64)
    vals = np.array([orc.decode(orc.E4M3, int(c)) for c in codes])
    enc = sa_synth.encode(vals, sa_synth.E4M3).astype(np.int64)
    same = (enc == codes) | ((codes == 0x80) & (enc == 0x80))
    assert same.all()
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * 40).astype(np.float32)
    x = x[np.abs(x) < 440]
    mine = sa_synth.encode(x.astype(np.float64), sa_synth.E4M3)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mine == theirs).all()
    b16 = sa_synth.encode(x.astype(np.float64), sa_synth.BF16)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (b16 == tb).all()


# -------------------------------------------------------------- visibility

def test_causal_pair_count_six_positions():
    # "Understanding LLMs" ch. 26 §26.4: causal length 6 allows 1+2+...+6 = 21 pairs (self included)
    g = golden("pair_counts.txt")
    n = int(g["n"])
    W = tiny(Q=np.zeros((1, 1, n, 1)), K=np.zeros((1, 1, n, 1)), V=np.zeros((1, 1, n, 1)), k=n)
    assert orc.count_visible(W) == g["causal_pairs"]
    assert orc.count_visible(W, causal=0) == n * n
    for n2 in (1, 7, 64):
        W2 = tiny(Q=np.zeros((1, 1, n2, 1)), K=np.zeros((1, 1, n2, 1)), V=np.zeros((1, 1, n2, 1)), k=n2)
        assert orc.count_visible(W2) == n2 * (n2 + 1) // 2


def test_window_candidate_pair_counts():
    # §26.4 example 26.3 and exercise 3: windows {i-1, i} -> 11 pairs, {i-2..i} -> 15 pairs
    # (per row 1,2,3,3,3,3).  Window index lists pass through the oracle's mask unchanged.
    g = golden("pair_counts.txt")
    n = int(g["n"])
    for width, key in ((2, "window2_pairs"), (3, "window3_pairs")):
        idx = np.array([[j if j >= 0 else -1 for j in range(i - width + 1, i + 1)] for i in range(n)], np.int32)
        Q = np.ones((1, 1, n, 1)); K = np.zeros((1, 1, n, 1)); V = np.ones((1, 1, n, 1))
        W = tiny(Q=Q, K=K, V=V, k=width)
        O, lse = orc.attend(W, idx)
        # equal logits: LSE = ln(count), so the per-row counts come back out of the softmax
        counts = np.rint(np.exp(lse[:, 0])).astype(int)
        assert counts.sum() == g[key]
        if width == 3:
            assert list(counts) == [int(x) for x in g["window3_rows"]]


# ------------------------------------------------------------ indexer score

def _hand_indexer():
    g = golden("indexer_hand.txt")
    q = np.array([[g["q0"], g["q1"]]])[None]  # [1,1,2,3]
    keys = np.array(g["keys"])[None]  # [1,4,3]
    w = np.array(g["w"])[None, None]
    return g, tiny(q_idx=q, k_idx=keys, w=w, causal=0, k=2)


def test_indexer_score_hand_worked_example():
    g, W = _hand_indexer()
    r = orc.scores(W)[0]
    assert np.array_equal(r, np.array(g["scores"]))
    W["w"] = np.array(g["w_neg"], dtype=np.float32)[None, None]
    assert np.array_equal(orc.scores(W)[0], np.array(g["scores_wneg"]))


def test_indexer_relu_identity_from_resmisa():
    # "PaperTrace 2.2 · Fine-grained indexing", §3.2 (ResMiSA): ReLU(z) = z + ReLU(-z).
    # Hence r(q) - r(-q) = sum_h w_h <q_h, k>, the unclipped linear term, computed here by
    # a plain matmul.  A dropped head, a sign slip or a transposed operand breaks it.
    rng = np.random.default_rng(3)
    B, n, H, d = 2, 40, 5, 16
    q = rand_f32(rng, (B, n, H, d)); kk = rand_f32(rng, (B, n, d))
    w = (rng.standard_normal((B, n, H))).astype(np.float32)  # any sign
    Wp = tiny(q_idx=q, k_idx=kk, w=w, causal=0)
    Wm = tiny(q_idx=-q, k_idx=kk, w=w, causal=0)
    diff = orc.scores(Wp) - orc.scores(Wm)
    lin = np.einsum("bih,bihd,bjd->bij", w.astype(np.float64), q.astype(np.float64), kk.astype(np.float64))
    assert np.allclose(diff, lin.reshape(B * n, n), rtol=1e-12, atol=1e-10)


def test_indexer_single_head_positive_reduces_to_dot_and_argsort():
    # One head, w = 1, all dot products positive: r = <q, k>, and the top-k is numpy's
    # stable descending argsort of the plain dot products.
    rng = np.random.default_rng(4)
    n, d, k = 50, 8, 7
    q = np.abs(rand_f32(rng, (1, n, 1, d))) + 0.1
    kk = np.abs(rand_f32(rng, (1, n, d))) + 0.1
    W = tiny(q_idx=q, k_idx=kk, w=np.ones((1, n, 1)), causal=0, k=k)
    r = orc.scores(W)
    dots = q[0, :, 0, :].astype(np.float64) @ kk[0].astype(np.float64).T
    assert np.allclose(r, dots, rtol=1e-12)
    idx, *_ = orc.select(W, r)
    for i in range(n):
        top = np.sort(np.argsort(-dots[i], kind="stable")[:k])
        assert np.array_equal(idx[i], top)


def test_indexer_positive_homogeneity():
    # ReLU(a z) = a ReLU(z) for a > 0: scaling k or w by a > 0 scales r by a, set unchanged.
    W = sa_synth.make_config(0)
    rows = np.arange(0, 256, 17, dtype=np.int32)
    base = orc.scores(W, rows)
    W2 = dict(W); W2["k_idx"] = (W["k_idx"] * np.float32(4.0)).astype(np.float32)
    W3 = dict(W); W3["w"] = (W["w"] * np.float32(0.5)).astype(np.float32)
    assert np.allclose(orc.scores(W2, rows), 4.0 * base, rtol=1e-12)
    assert np.allclose(orc.scores(W3, rows), 0.5 * base, rtol=1e-12)
    i1, *_ = orc.select(W, base, rows)
    i2, *_ = orc.select(W2, orc.scores(W2, rows), rows)
    assert np.array_equal(i1, i2)


@pytest.mark.parametrize("causal", [1, 0])
def test_indexer_brute_force_tiny_against_python_loops(causal):
    # Brute force in pure Python on a tiny problem with padding, causal and not.
    rng = np.random.default_rng(5)
    B, n, H, d = 2, 9, 3, 4
    q = rand_f32(rng, (B, n, H, d)); kk = rand_f32(rng, (B, n, d)); w = rng.random((B, n, H)).astype(np.float32)
    W = tiny(q_idx=q, k_idx=kk, w=w, causal=causal, kv_len=[9, 6])
    r = orc.scores(W).reshape(B, n, n)
    for b in range(B):
        for i in range(n):
            for j in range(n):
                vis = i < W["kv_len"][b] and j < W["kv_len"][b] and (j <= i or not causal)
                if not vis:
                    assert r[b, i, j] == -np.inf
                    continue
                tot = 0.0
                for h in range(H):
                    z = sum(float(q[b, i, h, t]) * float(kk[b, j, t]) for t in range(d))
                    tot += float(w[b, i, h]) * max(z, 0.0)
                assert abs(tot - r[b, i, j]) <= 1e-12 * max(1.0, abs(tot))


# ------------------------------------------------------------------ select

def test_select_hand_example_tie_goes_to_lower_position():
    g, W = _hand_indexer()
    r = orc.scores(W)
    idx, sk, skp1, nsel = orc.select(W, r, k=2)
    assert list(idx[0]) == [int(x) for x in g["select_k2"]]
    assert sk[0] == 2.0 and skp1[0] == 2.0  # the cutoff margin is zero: an exact tie
    idx3, *_ = orc.select(W, r, k=3)
    assert list(idx3[0]) == [int(x) for x in g["select_k3"]]


def test_select_tie_on_cobs_toy_keys():
    g = golden("tie_cobs_keys.txt")
    W = tiny(q_idx=np.array(g["q"])[None, None, None], k_idx=np.array(g["keys"])[None],
             w=np.ones((1, 1, 1)), causal=0, k=2)
    r = orc.scores(W)
    assert list(r[0]) == [float(x) for x in g["scores"]]
    idx, *_ = orc.select(W, r)
    assert list(idx[0]) == [int(x) for x in g["select_k2"]]


def test_select_matches_lexsort_with_many_ties():
    # Library routine: numpy lexsort by (position asc) within (score desc).
    rng = np.random.default_rng(6)
    n, k = 200, 37
    W = tiny(q_idx=np.zeros((1, n, 1, 1)), k_idx=np.zeros((1, n, 1)), w=np.zeros((1, n, 1)), causal=1, k=k)
    sc = rng.integers(0, 6, size=(n, n)).astype(np.float64)  # heavy exact ties
    sc[np.triu_indices(n, 1)] = -np.inf
    idx, sk, skp1, nsel = orc.select(W, sc)
    for i in range(n):
        vis = np.arange(i + 1)
        order = np.lexsort((vis, -sc[i, : i + 1]))
        want = np.sort(order[: min(k, i + 1)])
        got = idx[i][idx[i] >= 0]
        assert np.array_equal(got, want)
        assert nsel[i] == min(k, i + 1)


def test_select_causal_rows_shorter_than_k_are_padded_not_repeated():
    # Fine-grained indexing §2.1: with t < k only t+1 real positions exist; the other slots
    # are explicitly invalid, never repeats of position 0.
    W = sa_synth.make_config(0)
    idx, *_ = orc.select(W, orc.scores(W))
    for i in range(W["n_q"]):
        valid = idx[i][idx[i] >= 0]
        assert valid.size == min(W["k"], i + 1)
        assert np.array_equal(idx[i][: valid.size], valid)
        assert (idx[i][valid.size:] == -1).all()
        assert len(set(valid.tolist())) == valid.size
        if i < W["k"]:
            assert np.array_equal(valid, np.arange(i + 1))


def test_select_sliced_merge_equals_global():
    # Fine-grained indexing §2.1: slice the history, keep local top-k per slice, merge
    # keeping k of 2k; the result equals the global top-k.
    rng = np.random.default_rng(7)
    n, k = 300, 20
    W = tiny(q_idx=np.zeros((1, 1, 1, 1)), k_idx=np.zeros((1, n, 1)), w=np.zeros((1, 1, 1)), causal=0, k=k)
    sc = np.round(rng.standard_normal((1, n)) * 3, 1)  # some ties
    gidx, *_ = orc.select(W, sc)
    for slice_len in (1, 7, 64, 150, 300):
        cur = np.full((1, n), -np.inf)
        for s0 in range(0, n, slice_len):
            part = np.full((1, n), -np.inf)
            part[0, s0:s0 + slice_len] = sc[0, s0:s0 + slice_len]
            lidx, *_ = orc.select(W, part)
            both = cur.copy()
            keep = lidx[0][lidx[0] >= 0]
            both[0, keep] = sc[0, keep]
            m, *_ = orc.select(W, both)
            cur = np.full((1, n), -np.inf)
            mk = m[0][m[0] >= 0]
            cur[0, mk] = sc[0, mk]
        final = np.where(np.isfinite(cur[0]))[0]
        assert np.array_equal(final, gidx[0])


def test_select_stable_under_perturbation_below_half_margin():
    # Fine-grained indexing §3.1 eq. (9): if every score moves by less than delta_k / 2
    # the top-k set is unchanged.
    W = sa_synth.make_config(0)
    rows = all_rows(W)
    sc = orc.scores(W)
    idx, sk, skp1, nsel = orc.select(W, sc)
    rng = np.random.default_rng(8)
    for r in rows[rows >= W["k"]]:
        delta = sk[r] - skp1[r]
        assert delta >= 0
        if delta == 0:
            continue
        noise = rng.uniform(-0.49, 0.49, size=sc.shape[1]) * delta
        pert = sc[r:r + 1] + noise
        i2, *_ = orc.select(W, pert, rows=np.array([r], np.int32))
        assert np.array_equal(i2[0], idx[r])


# --------------------------------------------------------------- attention

def _attn_tiny(q, keys, vals, scale=1.0, causal=0):
    keys = np.asarray(keys, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    if vals.ndim == 1:
        vals = vals[:, None]
    Q = np.asarray(q, dtype=np.float64).reshape(1, 1, -1, keys.shape[-1])
    W = tiny(Q=Q, K=keys[None, None], V=vals[None, None], causal=causal, scale=scale, k=keys.shape[0])
    return W


def test_attention_lsh_toy_printed_numbers():
    g = golden("lsh_toy.txt")
    xs = [g["x1"], g["x2"], g["x3"], g["x4"]]
    W = _attn_tiny([g["x2"]], xs, np.eye(4))
    dots = [float(np.dot(np.float32(g["x2"]), np.float32(x))) for x in xs]
    for d_, key in zip(dots, ("dot_x1", "dot_x2", "dot_x3", "dot_x4")):
        assert abs(d_ - g[key]) < 1e-6
    O, lse = orc.attend(W, np.arange(4, dtype=np.int32)[None])
    assert abs(math.exp(lse[0, 0]) - g["expsum_all"]) <= g["expsum_tol"]
    O2, lse2 = orc.attend(W, np.array([[0, 1, -1, -1]], np.int32))
    kept = math.exp(lse2[0, 0] - lse[0, 0])
    assert abs((1 - kept) - g["dropped_mass"]) <= g["dropped_tol"]
    # V = identity exposes the probabilities; they sum to one
    assert abs(O[0, 0].sum() - 1.0) < 1e-12
    assert abs(O[0, 0][2:].sum() - g["dropped_mass"]) <= g["dropped_tol"]


def test_attention_kmeans_toy_printed_weights():
    g = golden("kmeans_toy.txt")
    ks = [g["k1"], g["k2"], g["k3"]]
    assert np.allclose(np.mean(ks, axis=0), g["mean_cluster1"])
    assert abs(np.dot(g["q"], g["k6p"]) - g["dot_k6p"]) < 1e-12
    W = _attn_tiny([g["q"]], ks, np.eye(3))
    O, lse = orc.attend(W, np.arange(3, dtype=np.int32)[None])
    assert np.allclose(O[0, 0], g["weights"], atol=g["weights_tol"])
    Wv = _attn_tiny([g["q"]], ks, g["v"])
    Ov, _ = orc.attend(Wv, np.arange(3, dtype=np.int32)[None])
    assert abs(Ov[0, 0, 0] - np.dot(g["weights"], g["v"])) < 3 * g["weights_tol"] * 4


def test_attention_cobs_block_mass_printed():
    g = golden("cobs_toy_block.txt")
    keys = g["keys"]
    for qk, lk, mk in (("q_a", "lnm_a", "m_a"), ("q_b", "lnm_b", "m_b"), ("q_c", "lnm_c", "m_c")):
        W = _attn_tiny([g[qk]], keys, np.ones(4))
        O, lse = orc.attend(W, np.arange(4, dtype=np.int32)[None])
        assert abs(lse[0, 0] - g[lk]) <= g["tol"]
        assert abs(math.exp(lse[0, 0]) - g[mk]) <= 1e-4 * g[mk]
        assert abs(O[0, 0, 0] - 1.0) < 1e-12  # softmax weights sum to one


def test_attention_linear_recursion_example_causal():
    # ch. 26 §26.5: logits ln(k_i) turn causal softmax attention into the printed running
    # weighted average S_i / Z_i: outputs 4, 2, 2.25, then 3.5 after appending (2, 6).
    g = golden("linear_recursion.txt")
    kw = list(g["key_weights"]) + [g["append_key"]]
    vals = list(g["values"]) + [g["append_value"]]
    n = len(kw)
    keys = np.log(np.array(kw))[:, None]
    Q = np.ones((1, 1, n, 1))
    W = tiny(Q=Q, K=keys[None, None], V=np.array(vals)[None, None, :, None], causal=1, scale=1.0, k=n)
    O, lse = orc.attend(W, full_idx(W))
    want = list(g["outputs"]) + [g["append_output"]]
    assert np.allclose(O[:, 0, 0], want, rtol=0, atol=1e-6)


def _torch_sdpa(Q, K, V, scale, mask):
    q = torch.from_numpy(Q.astype(np.float64)); k = torch.from_numpy(K.astype(np.float64))
    v = torch.from_numpy(V.astype(np.float64))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask),
                                                            scale=scale).numpy()


def test_attention_degenerate_full_set_equals_dense_causal_sdpa():
    # Spec invariant and Hashing-and-clustering §5.1 (minimal correctness tests):
    # when k >= the visible count, sparse attention equals dense causal attention.
    rng = np.random.default_rng(9)
    B, H, n, d = 2, 3, 24, 8
    Q, K, V = (rand_f32(rng, (B, H, n, d)) for _ in range(3))
    W = tiny(Q=Q, K=K, V=V, causal=1, scale=0.3, k=n)
    O, lse = orc.attend(W, full_idx(W))
    mask = np.tril(np.ones((n, n), dtype=bool))
    ref = _torch_sdpa(Q, K, V, 0.3, mask)  # [B,H,n,d]
    got = O.reshape(B, n, H, d).transpose(0, 2, 1, 3)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_gqa_sharing_matches_sdpa():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, n, d = 1, 6, 2, 16, 4
    Q = rand_f32(rng, (B, Hq, n, d)); K = rand_f32(rng, (B, Hkv, n, d)); V = rand_f32(rng, (B, Hkv, n, d))
    W = tiny(Q=Q, K=K, V=V, causal=1, scale=0.5, k=n)
    O, _ = orc.attend(W, full_idx(W))
    Kx = np.repeat(K, Hq // Hkv, axis=1); Vx = np.repeat(V, Hq // Hkv, axis=1)
    ref = _torch_sdpa(Q, Kx, Vx, 0.5, np.tril(np.ones((n, n), dtype=bool)))
    assert np.allclose(O.reshape(B, n, Hq, d).transpose(0, 2, 1, 3), ref, atol=1e-12)


def test_attention_local_window_equals_banded_sdpa():
    # Hashing and clustering §5.1: fixing the candidates to a local window must equal a
    # regular window implementation.
    rng = np.random.default_rng(11)
    n, d, width = 20, 5, 3
    Q, K, V = (rand_f32(rng, (1, 1, n, d)) for _ in range(3))
    W = tiny(Q=Q, K=K, V=V, causal=1, scale=0.7, k=width)
    idx = np.array([[j if j >= 0 else -1 for j in range(i - width + 1, i + 1)] for i in range(n)], np.int32)
    O, _ = orc.attend(W, idx)
    ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    mask = (jj <= ii) & (jj > ii - width)
    ref = _torch_sdpa(Q, K, V, 0.7, mask)
    assert np.allclose(O[:, 0, :], ref[0, 0], atol=1e-12)


def test_attention_block_mixture_and_exact_drop_error():
    # COBS reading note eq. (P3): o* = sum_b P_b v_b^c for any partition of the candidates
    # into blocks; eq. (2)-(3): renormalising over kept blocks S gives
    # o* - o_S = 1/(1 - tau) * sum_{b not in S} P_b (v_b^c - o*).
    rng = np.random.default_rng(12)
    n, d = 40, 6
    Q, K, V = (rand_f32(rng, (1, 1, n, d)) for _ in range(3))
    W = tiny(Q=Q, K=K, V=V, causal=0, scale=0.8, k=n)
    row = np.array([0], np.int32)
    o_all, lse_all = orc.attend(W, np.arange(n, dtype=np.int32)[None], rows=row)
    blocks = [np.arange(s, min(s + 7, n)) for s in range(0, n, 7)]
    P, vc = [], []
    for blk in blocks:
        ix = np.full((1, n), -1, np.int32); ix[0, : blk.size] = blk
        ob, lb = orc.attend(W, ix, rows=row)
        P.append(math.exp(lb[0, 0] - lse_all[0, 0])); vc.append(ob[0, 0])
    P, vc = np.array(P), np.array(vc)
    assert abs(P.sum() - 1) < 1e-12
    assert np.allclose((P[:, None] * vc).sum(0), o_all[0, 0], atol=1e-12)
    keep = [0, 2, 3]
    drop = [b for b in range(len(blocks)) if b not in keep]
    ix = np.full((1, n), -1, np.int32)
    sel = np.concatenate([blocks[b] for b in keep]); ix[0, : sel.size] = sel
    o_s, _ = orc.attend(W, ix, rows=row)
    tau = P[drop].sum()
    pred = (P[drop, None] * (vc[drop] - o_all[0, 0])).sum(0) / (1 - tau)
    assert np.allclose(o_all[0, 0] - o_s[0, 0], pred, atol=1e-12)


def test_attention_permutation_invariance_with_positions():
    # Hashing and clustering §5.2 (the permuted-order causal-leak test) and the north-star
    # invariant: permuting history storage together with its positions changes nothing;
    # causality and the tie-break use positions, not slots.
    W = sa_synth.make_config(0)
    rng = np.random.default_rng(13)
    perm = rng.permutation(W["n_kv"])  # slot s holds position perm[s]
    inv = np.argsort(perm)
    Wp = dict(W)
    Wp["k_idx"] = np.ascontiguousarray(W["k_idx"][:, perm])
    Wp["K"] = np.ascontiguousarray(W["K"][:, :, perm])
    Wp["V"] = np.ascontiguousarray(W["V"][:, :, perm])
    pos = perm[None].astype(np.int32)
    base = orc.select_attend(W)
    sc = orc.scores(Wp, pos_of_slot=pos)
    idx, *_ = orc.select(Wp, sc, pos_of_slot=pos)
    O, lse = orc.attend(Wp, idx, pos_of_slot=pos)
    mapped = np.where(idx >= 0, perm[np.maximum(idx, 0)], -1)
    assert np.array_equal(mapped, base["idx"])
    assert np.allclose(O, base["O"], atol=1e-12) and np.allclose(lse, base["lse"], atol=1e-12)
    assert inv.size == W["n_kv"]


def test_attention_ignores_invisible_and_invalid_indices():
    # Supplied indices that are -1, out of range, in the future or in the padding take no
    # part (Hashing and clustering §1.1: candidates intersect the causal and valid sets).
    rng = np.random.default_rng(14)
    n, d = 12, 4
    Q, K, V = (rand_f32(rng, (1, 1, n, d)) for _ in range(3))
    W = tiny(Q=Q, K=K, V=V, causal=1, scale=1.0, k=5, kv_len=[10])
    row = np.array([6], np.int32)
    clean, lc = orc.attend(W, np.array([[1, 4, 6, -1, -1]], np.int32), rows=row)
    dirty, ld = orc.attend(W, np.array([[1, 4, 6, 7, 11]], np.int32), rows=row)
    assert np.array_equal(clean, dirty) and np.array_equal(lc, ld)
    pad_row = np.array([10], np.int32)  # q_pos 10 >= kv_len: padded query row
    Op, lp = orc.attend(W, np.array([[0, 1, 2, 3, 4]], np.int32), rows=pad_row)
    assert (Op == 0).all() and np.isneginf(lp).all()


def test_padding_poison_never_leaks():
    # Padded history (positions >= kv_len) is filled with values that would dominate if read;
    # replacing them with other values changes nothing.
    W = sa_synth.make_config(1, n=256)
    rows = np.array([0, 100, 255, 256, 256 + W["kv_len"][1] - 1, 256 + W["kv_len"][1], 511], np.int32)
    a = orc.select_attend(W, rows)
    W2 = dict(W)
    for key in ("k_idx", "K", "V"):
        W2[key] = W[key].copy()
    L = W["kv_len"][1]
    W2["k_idx"][1, L:] = 0
    W2["K"][1, :, L:] = 0
    W2["V"][1, :, L:] = 0
    b = orc.select_attend(W2, rows)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["O"], b["O"])
    assert (a["idx"][-2:] == -1).all() and (a["O"][-2:] == 0).all() and np.isneginf(a["lse"][-2:]).all()


def test_kv_byte_accounting_example():
    # ch. 26 §26.2 example 26.1 / Table 26.1 and exercise 1: 2 * Hkv * d * n * bytes.
    g = golden("kv_bytes.txt")
    from bench import kv_cache_bytes  # the benchmark's own byte accounting
    d, n, b = int(g["head_dim"]), int(g["positions"]), int(g["bytes_per"])
    assert kv_cache_bytes(8, d, n, b) == g["mha_bytes"]
    assert kv_cache_bytes(2, d, n, b) == g["gqa2_bytes"]
    assert kv_cache_bytes(1, d, n, b) == g["mqa_bytes"]
    assert kv_cache_bytes(int(g["exercise_kv_heads"]), d, int(g["exercise_positions"]), b) == g["exercise_bytes"]


# ------------------------------------------------------------------ hierarchical selection
# "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the HISA paragraphs: score block
# representatives, keep k_b blocks, run the token indexer inside them, same top-k output.

HISA_CASES = {
    "causal_padded": dict(B=2, n_q=48, n_kv=64, Hidx=4, d_idx=64, k=8, lens=[64, 45]),
    "noncausal": dict(B=1, n_q=6, n_kv=96, Hidx=8, d_idx=32, k=12, causal=0, lens=[90]),
    "chunked": dict(B=2, n_q=20, n_kv=80, Hidx=4, d_idx=32, k=6, q_pos0=[40, 55], lens=[80, 80],
                    kidx_dtype=sa_synth.E4M3),
}


@pytest.mark.parametrize("case", list(HISA_CASES))
def test_hisa_keeping_every_block_is_the_flat_selection(case):
    # with k_b >= the number of blocks every visible position is a candidate, so the
    # hierarchical selection must be the flat token top-k
    kw = dict(HISA_CASES[case])
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    W = sa_synth.custom(seed=3, lens=lens, q_pos0=q_pos0, with_main=False, **kw)
    rows = all_rows(W)
    flat, _, _, _ = orc.select(W, orc.scores(W, rows), rows)
    for blk in (4, 8, 16):
        h = orc.hisa_select(W, blk, W["n_kv"] // blk + 2, rows)
        np.testing.assert_array_equal(h["idx"], flat)


def test_hisa_unit_blocks_reduce_to_the_flat_selection():
    # b = 1: a block is one key (bf16 keys round-trip exactly), so the block top-k_b with
    # k_b >= k already holds the token top-k and the second stage returns it
    W = sa_synth.custom(seed=5, B=2, n_q=40, n_kv=64, Hidx=4, d_idx=64, k=8, lens=[64, 33], with_main=False)
    rows = all_rows(W)
    flat, _, _, _ = orc.select(W, orc.scores(W, rows), rows)
    for kb in (8, 11):
        np.testing.assert_array_equal(orc.hisa_select(W, 1, kb, rows)["idx"], flat)


def test_bf16_rounding_of_block_means_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-3, 4, 4000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]])
    ref = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f64_to_bf16_bits(x), ref)


def _brute_hisa(q, kk, w, L, blk, kb, K):
    """Tiny-input brute force of the hierarchical selection for one query row, in plain
    Python floats with torch's bf16 rounding for the block means."""
    H, D = len(q), len(q[0])

    def score(key):
        return sum(w[h] * max(0.0, sum(q[h][d] * key[d] for d in range(D))) for h in range(H))

    P = L // blk
    blocks = []
    for B in range(P):
        mean = [sum(kk[B * blk + t][d] for t in range(blk)) / blk for d in range(D)]
        mean = torch.tensor(mean, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).tolist()
        blocks.append((-score(mean), B))
    keep = sorted(sorted(blocks)[:kb], key=lambda x: x[1])
    cand = [B * blk + t for _, B in keep for t in range(blk)] + list(range(P * blk, L))
    ranked = sorted((-score(kk[j]), j) for j in cand)
    return sorted(j for _, j in ranked[:K])


def test_hisa_matches_brute_force_on_tiny_rows():
    rng = np.random.default_rng(11)
    B, n_q, n_kv, H, D = 1, 10, 22, 3, 5
    q = rand_f32(rng, (B, n_q, H, D))
    kk = rand_f32(rng, (B, n_kv, D))
    w = rng.uniform(0, 1, (B, n_q, H)).astype(np.float32)
    for causal, q0 in ((1, 12), (0, 0)):
        W = tiny(q_idx=q, k_idx=kk, w=w, k=4, causal=causal, q_pos0=[q0], kv_len=[20])
        for blk, kb in ((3, 2), (4, 1), (2, 3)):
            got = orc.hisa_select(W, blk, kb)["idx"]
            for i in range(n_q):
                L = 0 if q0 + i >= 20 else (q0 + i + 1 if causal else 20)  # a row at or past kv_len sees nothing
                ref = _brute_hisa(q[0, i].astype(np.float64).tolist(), kk[0].astype(np.float64).tolist(),
                                  w[0, i].astype(np.float64).tolist(), L, blk, kb, 4)
                assert got[i, : len(ref)].tolist() == ref and (got[i, len(ref):] == -1).all(), (causal, blk, kb, i)


def test_hisa_misses_a_strong_token_inside_a_weak_block():
    # a coarse miss cannot be recovered by the token stage: position 9 scores highest, but
    # its block's mean is low, so with one block kept (and no open block) it is not selected
    D = 2
    kk = np.zeros((1, 12, D))
    kk[0, 0:4] = [1.0, 0.0]          # block 0: uniformly good keys, mean score 1
    kk[0, 4:8] = [0.25, 0.0]         # block 1: weak
    kk[0, 8:12] = [-3.0, 0.0]        # block 2: very negative keys ...
    kk[0, 9] = [5.0, 0.0]            # ... and one strong token (block mean still negative)
    q = np.array([[[[1.0, 0.0]]]])
    w = np.ones((1, 1, 1))
    W = tiny(q_idx=q, k_idx=kk, w=w, k=2, causal=0)
    flat, _, _, _ = orc.select(W, orc.scores(W))
    assert flat[0].tolist() == [0, 9]  # ties among block 0 go to the lowest position
    h = orc.hisa_select(W, 4, 1)
    assert h["blocks"][0].tolist() == [0]
    assert h["idx"][0].tolist() == [0, 1]
    assert orc.hisa_select(W, 4, 3)["idx"][0].tolist() == [0, 9]


# ------------------------------------------------------------------ active index heads
# "PaperTrace 2.2 · Fine-grained indexing", §1.1 and §2.2, the MISA paragraphs: route each query to g of
# its G index heads by the block-averaged |weighted ReLU| response, score with those only.

@pytest.mark.parametrize("case", list(HISA_CASES))
def test_misa_with_every_head_active_is_the_flat_selection(case):
    kw = dict(HISA_CASES[case])
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    W = sa_synth.custom(seed=8, lens=lens, q_pos0=q_pos0, with_main=False, **kw)
    rows = all_rows(W)
    flat, _, _, _ = orc.select(W, orc.scores(W, rows), rows)
    np.testing.assert_array_equal(orc.misa_select(W, 8, W["Hidx"], rows)["idx"], flat)


def _brute_misa(q, kk, w, L, blk, g, K):
    """Tiny-input brute force of the active-head selection for one query row."""
    H, D = len(q), len(q[0])
    dot = lambda a, b: sum(x * y for x, y in zip(a, b))
    P = L // blk
    means = []
    for B in range(P):
        m = [sum(kk[B * blk + t][d] for t in range(blk)) / blk for d in range(D)]
        means.append(torch.tensor(m, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).tolist())
    route = [abs(w[h]) * (sum(max(0.0, dot(q[h], mb)) for mb in means) / P if P else 0.0) for h in range(H)]
    heads = sorted(h for _, h in sorted((-route[h], h) for h in range(H))[:g])
    sc = [(-sum(w[h] * max(0.0, dot(q[h], kk[j])) for h in heads), j) for j in range(L)]
    return heads, sorted(j for _, j in sorted(sc)[:K])


def test_misa_matches_brute_force_on_tiny_rows():
    rng = np.random.default_rng(17)
    B, n_q, n_kv, H, D = 1, 9, 20, 5, 4
    q = rand_f32(rng, (B, n_q, H, D))
    kk = rand_f32(rng, (B, n_kv, D))
    w = rng.uniform(-1, 1, (B, n_q, H)).astype(np.float32)  # a negative weight routes by |w|
    for causal, q0 in ((1, 2), (0, 0)):
        W = tiny(q_idx=q, k_idx=kk, w=w, k=3, causal=causal, q_pos0=[q0], kv_len=[18])
        for blk, g in ((3, 2), (4, 1), (2, 3)):
            got = orc.misa_select(W, blk, g)
            for i in range(n_q):
                L = 0 if q0 + i >= 18 else (q0 + i + 1 if causal else 18)
                heads, ref = _brute_misa(q[0, i].astype(np.float64).tolist(), kk[0].astype(np.float64).tolist(),
                                         w[0, i].astype(np.float64).tolist(), L, blk, g, 3)
                if L == 0:
                    assert (got["idx"][i] == -1).all()
                    continue
                assert got["heads"][i].tolist() == heads, (causal, blk, g, i)
                assert got["idx"][i, : len(ref)].tolist() == ref and (got["idx"][i, len(ref):] == -1).all()


def test_misa_routes_to_the_head_with_the_larger_weighted_block_response():
    # head 0 matches block 0 only, head 1 matches both blocks, head 2 never fires; with the
    # same weights head 1 wins; a 3x weight on head 0 makes it win (mean 3 * 0.5 > 1)
    kk = np.array([[[1.0, 0.0]] * 4 + [[0.0, 1.0]] * 4])
    q = np.array([[[[1.0, 0.0], [1.0, 1.0], [-1.0, -1.0]]]])
    W = tiny(q_idx=q, k_idx=kk, w=np.ones((1, 1, 3)), k=2, causal=0)
    r = orc.misa_select(W, 4, 1)
    np.testing.assert_allclose(r["route"][0], [0.5, 1.0, 0.0])
    assert r["heads"][0].tolist() == [1]
    W2 = tiny(q_idx=q, k_idx=kk, w=np.array([[[3.0, 1.0, 1.0]]]), k=2, causal=0)
    r2 = orc.misa_select(W2, 4, 1)
    assert r2["heads"][0].tolist() == [0]
    assert r2["idx"][0].tolist() == [0, 1]  # head 0 scores block 0's keys 3, the rest 0: lowest positions


# ------------------------------------------------------------------ paged K/V
# "PaperTrace 2.2 · Fine-grained indexing", §2.1 (the main-KV gather reaches physical rows
# through the block table) and §3.1 (block_table maps logical positions to physical pages).


@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_paged_attention_on_a_shuffled_pool_equals_the_contiguous_layout(page_size):
    # Paging is a storage layout: scattering every batch's rows to random pages of a pool
    # (unused rows poisoned) and attending through the table must give exactly the result on
    # the contiguous tensors.  A wrong page or offset formula reads another row or a poison row.
    W = sa_synth.custom(seed=21, B=2, n_q=40, n_kv=150, Hq=2, Hkv=2, d_qk=64, d_v=64, k=24, lens=[150, 97])
    rows = all_rows(W)
    ref = orc.select_attend(W, rows)
    bt, pool_rows = sa_synth.paged_layout(5, W["B"], W["n_kv"], page_size)
    fill = sa_synth.encode(np.array([sa_synth.poison_value(W["main_dtype"])]), W["main_dtype"])[0]
    Kp = sa_synth.to_pool(W["K"], bt, page_size, pool_rows, fill)
    Vp = sa_synth.to_pool(W["V"], bt, page_size, pool_rows, fill)
    O, lse = orc.attend_paged(W, ref["idx"], Kp, Vp, bt, page_size, rows)
    assert np.array_equal(O, ref["O"]) and np.array_equal(lse, ref["lse"])


def test_paged_attention_latent_layout_and_page_order():
    # Latent layout (V = the first d_v columns of each K row) through pages; a table whose
    # pages are listed in reverse order for batch 0 is followed, not the pool order.
    W = sa_synth.make_config(3, B=2, n_kv=300, k=64)
    rows = all_rows(W)
    ref = orc.select_attend(W, rows)
    ps = 32
    npg = -(-W["n_kv"] // ps)
    bt = np.stack([np.arange(npg)[::-1], npg + np.arange(npg)]).astype(np.int32)
    Kp = sa_synth.to_pool(W["K"], bt, ps, 2 * npg * ps, 0)
    O, lse = orc.attend_paged(W, ref["idx"], Kp, None, bt, ps, rows)
    assert np.array_equal(O, ref["O"]) and np.array_equal(lse, ref["lse"])
    # reading the pool as if it were contiguous (identity table) is a different, wrong answer
    ident = np.stack([np.arange(npg), npg + np.arange(npg)]).astype(np.int32)
    O2, _ = orc.attend_paged(W, ref["idx"], Kp, None, ident, ps, rows)
    assert not np.allclose(O2[0], ref["O"][0])


def test_paged_attention_hand_case_page_outside_the_pool_is_skipped():
    # Six positions in pages of two; the pool holds three pages, stored in the order
    # (page 1, page 2, page 0).  Position 3 lives on logical page 1 = pool page 0, row 1.
    rng = np.random.default_rng(22)
    Q, K, V = (rand_f32(rng, (1, 1, 6, 4)) for _ in range(3))
    W = tiny(Q=Q, K=K, V=V, causal=0, scale=0.5, k=4)
    bt = np.array([[2, 0, 1]], np.int32)
    Kp = np.empty((1, 6, 4), np.float32)
    Vp = np.empty((1, 6, 4), np.float32)
    for j in range(6):
        r = bt[0, j // 2] * 2 + j % 2
        Kp[0, r], Vp[0, r] = K[0, 0, j], V[0, 0, j]
    assert np.array_equal(Kp[0, 1], K[0, 0, 3])
    row = np.array([4], np.int32)
    idx = np.array([[0, 3, 4, 5]], np.int32)
    O, lse = orc.attend_paged(W, idx, Kp, Vp, bt, 2, rows=row)
    Oc, lc = orc.attend(W, idx, rows=row)
    assert np.array_equal(O, Oc) and np.array_equal(lse, lc)
    # page 2 (positions 4, 5) pointed outside the pool: those candidates drop out
    bad = bt.copy()
    bad[0, 2] = 3
    Ob, lb = orc.attend_paged(W, idx, Kp, Vp, bad, 2, rows=row)
    Oe, le = orc.attend(W, np.array([[0, 3, -1, -1]], np.int32), rows=row)
    assert np.array_equal(Ob, Oe) and np.array_equal(lb, le)


# ------------------------------------------------------------------ grouped candidate sets
# "PaperTrace 2.2 · Fine-grained indexing", §2 eq. (5): G groups of main heads, one selector
# per group; G = 1 is the shared set, G = Hq gives every head its own set.


def _per_head_brute(W, rows):
    """Every head its own selector and softmax, in pure Python (tiny sizes): index head h
    scores w_h ReLU(<q_h, k_s>), the k best visible positions (ties to the lower position),
    query head h attends over them."""
    B, nq, k = W["B"], W["n_q"], W["k"]
    q, kk, w = W["q_idx"].astype(np.float64), W["k_idx"].astype(np.float64), W["w"].astype(np.float64)
    Q, K, V = W["Q"].astype(np.float64), W["K"].astype(np.float64), W["V"].astype(np.float64)
    outO = np.zeros((len(rows), W["Hq"], W["d_v"]))
    sets = []
    for n, row in enumerate(rows):
        b, i = divmod(int(row), nq)
        L = i + 1 if W["causal"] else W["n_kv"]
        per = []
        for h in range(W["Hq"]):
            sc = [w[b, i, h] * max(0.0, sum(q[b, i, h, d] * kk[b, s, d] for d in range(W["d_idx"]))) for s in range(L)]
            order = sorted(range(L), key=lambda s: (-sc[s], s))[:k]
            per.append(sorted(order))
            hk = h // (W["Hq"] // W["Hkv"])
            logits = [W["scale"] * sum(Q[b, h, i, d] * K[b, hk, s, d] for d in range(W["d_qk"])) for s in order]
            m = max(logits)
            e = [math.exp(x - m) for x in logits]
            for s, ev in zip(order, e):
                outO[n, h] += ev / sum(e) * V[b, hk, s]
        sets.append(per)
    return sets, outO


def test_grouped_sets_one_group_is_the_shared_selection():
    W = sa_synth.custom(seed=41, B=2, n_q=30, n_kv=50, Hq=4, Hkv=4, d_qk=64, d_v=64, Hidx=8, d_idx=32, k=8,
                        lens=[50, 37], main_dtype=sa_synth.F32, qidx_dtype=sa_synth.F32, kidx_dtype=sa_synth.F32)
    rows = all_rows(W)
    idx, O, lse = orc.select_attend_grouped(W, 1, rows)
    ref = orc.select_attend(W, rows)
    assert np.array_equal(idx[0], ref["idx"]) and np.array_equal(O, ref["O"]) and np.array_equal(lse, ref["lse"])


def test_grouped_sets_one_head_per_group_is_a_per_head_brute_force():
    rng = np.random.default_rng(42)
    B, n, H, d, di = 1, 9, 3, 4, 3
    W = tiny(Q=rand_f32(rng, (B, H, n, d)), K=rand_f32(rng, (B, H, n, d)), V=rand_f32(rng, (B, H, n, d)),
             q_idx=rand_f32(rng, (B, n, H, di)), k_idx=rand_f32(rng, (B, n, di)),
             w=rng.uniform(0.2, 1.0, (B, n, H)), k=3, causal=1, scale=0.5)
    rows = all_rows(W)
    idx, O, _ = orc.select_attend_grouped(W, H, rows)
    sets, O_bf = _per_head_brute(W, rows)
    for n_, row in enumerate(rows):
        for h in range(H):
            got = sorted(int(x) for x in idx[h, n_] if x >= 0)
            assert got == sets[n_][h], (row, h)
    assert np.allclose(O, O_bf, atol=1e-12)


def test_grouped_sets_hand_case_each_group_follows_its_index_heads():
    # Two groups, one index head each.  Index head 0 matches key 1 only, index head 1 key 3
    # only; with k = 1 group 0's query heads see position 1 and group 1's position 3, so
    # each output is that position's value row exactly.
    n, d = 5, 2
    kk = np.zeros((1, n, 2)); kk[0, 1] = [1, 0]; kk[0, 3] = [0, 1]
    qi = np.zeros((1, n, 2, 2)); qi[0, :, 0] = [1, 0]; qi[0, :, 1] = [0, 1]
    V = np.arange(1 * 2 * n * d, dtype=np.float64).reshape(1, 2, n, d)
    W = tiny(Q=np.ones((1, 2, n, d)), K=np.ones((1, 2, n, d)), V=V, q_idx=qi, k_idx=kk, w=np.ones((1, n, 2)),
             k=1, causal=0)
    idx, O, lse = orc.select_attend_grouped(W, 2, np.array([4], np.int32))
    assert idx[0, 0, 0] == 1 and idx[1, 0, 0] == 3
    assert np.array_equal(O[0, 0], V[0, 0, 1]) and np.array_equal(O[0, 1], V[0, 1, 3])
    assert np.allclose(lse, 2.0)  # one logit <1,1>·<1,1> = 2 at scale 1


def test_grouped_sets_swapping_groups_swaps_the_outputs():
    W = sa_synth.custom(seed=43, B=1, n_q=24, n_kv=40, Hq=4, Hkv=1, d_qk=64, d_v=64, Hidx=8, d_idx=32, k=6,
                        main_dtype=sa_synth.F32, qidx_dtype=sa_synth.F32, kidx_dtype=sa_synth.F32)
    rows = all_rows(W)
    idx, O, lse = orc.select_attend_grouped(W, 2, rows)
    Ws = dict(W)
    Ws["q_idx"] = np.ascontiguousarray(np.concatenate([W["q_idx"][:, :, 4:], W["q_idx"][:, :, :4]], axis=2))
    Ws["w"] = np.ascontiguousarray(np.concatenate([W["w"][:, :, 4:], W["w"][:, :, :4]], axis=2))
    Ws["Q"] = np.ascontiguousarray(np.concatenate([W["Q"][:, 2:], W["Q"][:, :2]], axis=1))
    idx2, O2, lse2 = orc.select_attend_grouped(Ws, 2, rows)
    assert np.array_equal(idx2[0], idx[1]) and np.array_equal(idx2[1], idx[0])
    assert np.array_equal(O2[:, :2], O[:, 2:]) and np.array_equal(lse2[:, 2:], lse[:, :2])
    assert not np.array_equal(idx[0], idx[1])  # the two groups really select differently


# ---------------------------------------------------------------- shared linear term + residual heads
# "PaperTrace 2.2 · Fine-grained indexing", §2.2 (ResMiSA): ReLU(z) = z + ReLU(-z) turns the
# heads' linear terms into one shared dot product; the residual ReLU(-z) runs on some heads.

@pytest.mark.parametrize("case", list(HISA_CASES))
def test_resmisa_with_every_head_residual_is_the_flat_score(case):
    # every head keeps its residual: shared linear term + all residuals = the indexer's own
    # score (the C oracle's, computed head by head), to rounding
    kw = dict(HISA_CASES[case])
    lens, q_pos0 = kw.pop("lens", None), kw.pop("q_pos0", None)
    W = sa_synth.custom(seed=9, lens=lens, q_pos0=q_pos0, with_main=False, **kw)
    rows = all_rows(W)
    flat = orc.scores(W, rows)
    heads = np.tile(np.arange(W["Hidx"], dtype=np.int32), (rows.size, 1))
    res = orc.resmisa_scores(W, heads, rows)
    fin = np.isfinite(flat)
    assert np.array_equal(fin, np.isfinite(res))
    scale = np.abs(flat[fin]).max()
    assert np.abs(res[fin] - flat[fin]).max() <= 1e-12 * scale
    r = orc.resmisa_select(W, 8, W["Hidx"], rows)
    ref, sk, skp1, _ = orc.select(W, flat, rows)
    # the selections agree wherever the cutoff margin is above the rounding
    ok = (sk - skp1) > 1e-9 * scale
    assert ok.sum() > rows.size // 2
    np.testing.assert_array_equal(r["idx"][ok], ref[ok])


def test_resmisa_hand_case_keeps_the_inactive_heads_linear_term():
    # two heads, q1 = (1, 0), q2 = (0, 1), w = (1, 2); keys k0 = (1, -1), k1 = (-1, 1), k2 = (2, 2)
    # flat r = w1 ReLU(z1) + w2 ReLU(z2):          k0: 1,  k1: 2,  k2: 6
    # residual on head 2 only: (z1 + 2 z2) + 2 ReLU(-z2): k0: -1 + 2 = 1, k1: 1 + 0 = 1, k2: 6
    #   (head 1 is inactive: its linear term z1 replaces ReLU(z1), exact for z1 >= 0, -1 for k1)
    # residual on head 1 only: (z1 + 2 z2) + ReLU(-z1):   k0: -1 + 0 = -1, k1: 1 + 1 = 2, k2: 6
    # no residual (shared linear term only):             k0: -1, k1: 1, k2: 6
    q = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    kk = np.array([[[1.0, -1.0], [-1.0, 1.0], [2.0, 2.0]]])
    W = tiny(q_idx=q, k_idx=kk, w=np.array([[[1.0, 2.0]]]), k=2, causal=0)
    np.testing.assert_allclose(orc.scores(W)[0], [1.0, 2.0, 6.0])
    np.testing.assert_allclose(orc.resmisa_scores(W, [[1]])[0], [1.0, 1.0, 6.0])
    np.testing.assert_allclose(orc.resmisa_scores(W, [[0]])[0], [-1.0, 2.0, 6.0])
    np.testing.assert_allclose(orc.resmisa_scores(W, np.zeros((1, 0), np.int32))[0], [-1.0, 1.0, 6.0])
    # top 2: with head 2's residual k0 and k1 tie at 1 (lower position wins) -> {0, 2}
    assert orc.resmisa_select(W, 1, 1, heads=[[1]])["idx"][0].tolist() == [0, 2]
    assert orc.resmisa_select(W, 1, 1, heads=[[0]])["idx"][0].tolist() == [1, 2]


def _brute_resmisa(q, kk, w, L, heads, K):
    dot = lambda a, b: sum(x * y for x, y in zip(a, b))
    H = len(q)
    sc = []
    for j in range(L):
        z = [dot(q[h], kk[j]) for h in range(H)]
        lin = sum(w[h] * z[h] for h in range(H))
        sc.append((-(lin + sum(w[h] * max(0.0, -z[h]) for h in heads)), j))
    return sorted(j for _, j in sorted(sc)[:K])


def test_resmisa_matches_brute_force_on_tiny_rows():
    rng = np.random.default_rng(19)
    B, n_q, n_kv, H, D = 1, 9, 20, 5, 4
    q = rand_f32(rng, (B, n_q, H, D))
    kk = rand_f32(rng, (B, n_kv, D))
    w = rng.uniform(-1, 1, (B, n_q, H)).astype(np.float32)
    for causal, q0 in ((1, 2), (0, 0)):
        W = tiny(q_idx=q, k_idx=kk, w=w, k=3, causal=causal, q_pos0=[q0], kv_len=[18])
        # g < H: with every head residual, scores that the flat formula makes exactly 0 come
        # out as +-1e-16 (linear term plus residual), so exact ties there break by rounding
        for blk, g in ((3, 2), (4, 1), (2, 4)):
            got = orc.resmisa_select(W, blk, g)
            mis = orc.misa_select(W, blk, g)
            for i in range(n_q):
                L = 0 if q0 + i >= 18 else (q0 + i + 1 if causal else 18)
                if L == 0:
                    assert (got["idx"][i] == -1).all()
                    continue
                assert got["heads"][i].tolist() == mis["heads"][i].tolist()  # the MISA routing
                ref = _brute_resmisa(q[0, i].astype(np.float64).tolist(), kk[0].astype(np.float64).tolist(),
                                     w[0, i].astype(np.float64).tolist(), L, got["heads"][i].tolist(), 3)
                assert got["idx"][i, : len(ref)].tolist() == ref and (got["idx"][i, len(ref):] == -1).all()
