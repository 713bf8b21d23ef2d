"""GPU edge cases: degenerate sizes, empty and padded histories, exact ties, chunked
prefill, non-finite inputs, every attention kernel variant, arbitrary caller indices."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from tests.checker import check_index_rows
from token_selector_gather_amd.inputs import device_workload
from tests.device_inputs import empty_outputs

pytestmark = pytest.mark.gpu
BF16, F32, E4M3 = sa_synth.BF16, sa_synth.F32, sa_synth.E4M3


def _print(x):
    print(x, flush=True)


@pytest.mark.parametrize("name,kw", [
    ("k_exceeds_history", dict(n_q=100, n_kv=100, k=300)),
    ("single_row_single_key", dict(n_q=1, n_kv=1, k=4)),
    ("chunked_prefill_qpos0", dict(B=2, n_q=64, n_kv=300, k=40, q_pos0=[236, 100], lens=[300, 180])),
    ("empty_and_padded_batches", dict(B=3, n_q=48, n_kv=96, k=24, lens=[96, 0, 37])),
    ("noncausal_padded", dict(B=2, n_q=20, n_kv=200, k=33, causal=0, lens=[200, 77])),
    ("mha_d64", dict(n_q=80, n_kv=80, d_qk=64, d_v=64, k=20)),
    ("mha_d256", dict(n_q=70, n_kv=70, d_qk=256, d_v=256, Hq=1, Hkv=1, k=50)),
    ("gqa_g2_d64", dict(n_q=64, n_kv=64, Hq=4, Hkv=2, d_qk=64, d_v=64, k=12)),
    ("gqa_g4_f32", dict(n_q=50, n_kv=50, Hq=4, Hkv=1, d_qk=32, d_v=32, k=10, main_dtype=F32, qidx_dtype=F32,
                        kidx_dtype=F32)),
    ("f32_index_bf16_main", dict(n_q=40, n_kv=40, k=8, qidx_dtype=F32, kidx_dtype=F32)),
    ("bf16_q_e4m3_k_h16", dict(n_q=96, n_kv=96, Hidx=16, d_idx=32, k=20, kidx_dtype=E4M3)),
    ("bf16_q_e4m3_k_h32", dict(n_q=96, n_kv=96, Hidx=32, d_idx=128, k=20, kidx_dtype=E4M3)),
    ("index_h4_d32", dict(n_q=100, n_kv=100, Hidx=4, d_idx=32, k=30)),
    ("index_h2_plain_path", dict(n_q=33, n_kv=33, Hidx=2, d_idx=16, k=5)),
    ("mla_g16_separate_v", dict(n_q=40, n_kv=300, Hq=16, Hkv=1, d_qk=576, d_v=512, k=64, mla=False,
                                q_pos0=[260], lens=[300])),
    ("mla_g128_aliased_v", dict(n_q=6, n_kv=500, Hq=128, Hkv=1, d_qk=576, d_v=512, k=100, mla=True,
                                q_pos0=[494], lens=[500])),
    ("mla_two_kv_heads", dict(n_q=30, n_kv=130, Hq=32, Hkv=2, d_qk=576, d_v=512, k=45, mla=False,
                              q_pos0=[100], lens=[130])),
    ("mla_g32_aliased_v", dict(n_q=12, n_kv=900, Hq=32, Hkv=1, d_qk=576, d_v=512, k=230, mla=True,
                               q_pos0=[888], lens=[900])),
    ("mla_g64_aliased_v_two_rows", dict(B=2, n_q=10, n_kv=700, Hq=64, Hkv=1, d_qk=576, d_v=512, k=150, mla=True,
                                        q_pos0=[650, 90], lens=[660, 100])),
])
def test_edge_case_end_to_end(name, kw):
    _print("edge " + name)
    W = sa_synth.custom(**kw)
    gc.full_check(W)


def test_all_keys_identical_selects_lowest_positions():
    W = sa_synth.custom(B=1, n_q=64, n_kv=64, k=10, causal=1)
    W["k_idx"][:] = W["k_idx"][0, 0]
    idx, O, lse, st = gc.gpu_select_attend(W)
    assert st == sa.SA_OK
    for i in range(64):
        m = min(10, i + 1)
        assert list(idx[0, i, :m]) == list(range(m)) and (idx[0, i, m:] == -1).all()
    gc.full_check(W, tie_groups={0: [list(range(64))]})


def test_nonfinite_index_input_sets_device_status_then_clears():
    W = sa_synth.custom(B=1, n_q=32, n_kv=32, k=8)
    W["q_idx"] = W["q_idx"].copy()
    W["q_idx"][0, 20, 1, 3] = 0x7FC0  # bf16 NaN
    _, _, _, st = gc.gpu_select_attend(W)
    assert st == sa.SA_ERR_NONFINITE
    # the status word was cleared by the read: a clean call on the same workspace reports OK
    P, d = device_workload(W)
    ws = sa.workspace(P, sa.SA_OP_SELECT_ATTEND)
    O, lse, idx = empty_outputs(W, torch.bfloat16)
    d["q_idx"][0, 20, 1, 3] = float("nan")
    sa.sa_select_attend(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse, ws)
    assert sa.sa_device_status(ws) == sa.SA_ERR_NONFINITE
    d["q_idx"][0, 20, 1, 3] = 1.0
    sa.sa_select_attend(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse, ws)
    assert sa.sa_device_status(ws) == sa.SA_OK


def test_nan_in_e4m3_index_key_is_reported():
    W = sa_synth.custom(B=1, n_q=16, n_kv=64, k=8, kidx_dtype=E4M3, Hidx=8, d_idx=64, causal=0)
    W["k_idx"] = W["k_idx"].copy()
    W["k_idx"][0, 5, 7] = 0x7F
    _, _, _, st = gc.gpu_select_attend(W)
    assert st == sa.SA_ERR_NONFINITE


@pytest.mark.parametrize("kw", [dict(), dict(Hq=128, Hkv=1, d_qk=576, d_v=512, mla=True)])
def test_sparse_attn_ignores_invalid_caller_indices(kw):
    # -1, out of range, future (causal) and padded entries are skipped; order is irrelevant
    W = sa_synth.custom(B=1, n_q=40, n_kv=64, k=24, lens=[50], **kw)
    rng = np.random.default_rng(0)
    idx = np.full((1, 40, 24), -1, np.int32)
    for i in range(40):
        vis = rng.permutation(i + 1)[: min(10, i + 1)]
        junk = [-1, 64, 1 << 20, i + 1, i + 5, 55, 63]
        row = np.concatenate([vis, junk[: 24 - vis.size]])
        idx[0, i, : row.size] = rng.permutation(row)
    O, lse = gc.gpu_sparse_attn(W, idx)
    rows = np.arange(40, dtype=np.int32)
    O_or, lse_or = orc.attend(W, idx.reshape(40, 24), rows)
    gc.compare_attention(W, rows, O, lse, O_or, lse_or)


def test_sparse_attn_empty_candidate_rows_give_zero_and_neg_inf():
    W = sa_synth.custom(B=1, n_q=8, n_kv=16, k=4, Hq=128, Hkv=1, d_qk=576, d_v=512, mla=True)
    idx = np.full((1, 8, 4), -1, np.int32)
    O, lse = gc.gpu_sparse_attn(W, idx)
    assert (O == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("Hq", [32, 64, 128])
def test_mla_logits_far_above_the_first_tile_rerun_the_set(Hq):
    """The latent kernel fixes each head's reference maximum at its first tile of
    candidates; a later logit more than 64 (log2 units) above it makes the kernel run the
    set again against the true maximum.  Low positions get small keys and the queries are
    scaled up, so every head takes that second run."""
    _print("mla second run Hq=%d" % Hq)
    W = sa_synth.custom(B=1, n_q=4, n_kv=400, k=160, Hq=Hq, Hkv=1, d_qk=576, d_v=512, mla=True,
                        q_pos0=[396], lens=[400])
    K = sa_synth.bf16_to_f32(W["K"]).astype(np.float64)
    K[:, :, :200, :] *= 0.01
    W["K"] = sa_synth.encode(K, BF16)
    W["Q"] = sa_synth.encode(sa_synth.bf16_to_f32(W["Q"]).astype(np.float64) * 100.0, BF16)
    rows = np.arange(4, dtype=np.int32)
    # every set starts below position 200 and reaches past it, where logits are far above
    # the first tile's
    idx = np.stack([np.arange(100 + 20 * i, 260 + 20 * i, dtype=np.int32) for i in range(4)])
    O, lse = gc.gpu_sparse_attn(W, idx.reshape(1, 4, 160))
    O_or, lse_or = orc.attend(W, idx, rows)
    assert lse_or.min() > 50
    gc.compare_attention(W, rows, O, lse, O_or, lse_or)


def test_tile_attention_skips_unselected_tiles_and_ignores_order():
    # bf16 MHA d = 128 with 64 k >= 2 n_kv takes the tile kernel.  Caller lists that touch
    # only two of the eight 64-key tiles (the others must be skipped), in descending order,
    # mixed with -1, out-of-range and invisible entries, against the oracle.
    W = sa_synth.custom(seed=71, B=2, n_q=130, n_kv=512, Hq=2, Hkv=2, d_qk=128, d_v=128, k=32, causal=1,
                        q_pos0=np.array([382, 300], np.int32), lens=[512, 430])
    rng = np.random.default_rng(72)
    R = W["B"] * W["n_q"]
    idx = np.full((R, W["k"]), -1, np.int32)
    for r in range(R):
        cand = np.concatenate([np.arange(64, 128), np.arange(256, 320)])
        pick = rng.choice(cand, 24, replace=False)
        row = np.concatenate([np.sort(pick)[::-1], [-1, 9999, -5, 600, -1, -1, -1, -1]])
        idx[r] = row.astype(np.int32)
    rows = np.arange(R, dtype=np.int32)
    O, lse = gc.gpu_sparse_attn(W, idx.reshape(W["B"], W["n_q"], -1))
    O_or, lse_or = orc.attend(W, idx, rows)
    gc.compare_attention(W, rows, O, lse, O_or, lse_or)


@pytest.mark.parametrize("hidx,didx,kdt", [(16, 64, E4M3), (32, 128, BF16), (64, 128, E4M3)])
def test_decode_selection_fills_its_first_digit_in_the_index_scan(hidx, didx, kdt):
    # Few long rows take the sliced top-k, whose first radix digit the index scan adds while it
    # writes the scores: the selection still matches the oracle, a row shorter than k lists all
    # its positions, a NaN key at a visible position is reported and one past kv_len is not read.
    def work():
        return sa_synth.custom(seed=71 + hidx, B=3, n_q=1, n_kv=9000, Hq=2, Hkv=2, d_qk=64, d_v=64, Hidx=hidx,
                               d_idx=didx, kidx_dtype=kdt, k=256, lens=[9000, 8500, 200], q_pos0=[8999, 8499, 199])
    W = work()
    rows = np.arange(3, dtype=np.int32)
    idx, _, _, st = gc.gpu_select_attend(W)
    assert st == sa.SA_OK
    ref_sc = orc.scores(W, rows)
    ref_idx, sk, _, _ = orc.select(W, ref_sc, rows)
    check_index_rows(W, rows, idx.reshape(3, -1), ref_sc, ref_idx, sk)
    assert list(idx[2, 0, :200]) == list(range(200)) and (idx[2, 0, 200:] == -1).all()
    gc.full_check(W)
    for b, j, want in [(0, 1234, sa.SA_ERR_NONFINITE), (1, 8700, sa.SA_OK)]:
        W = work()
        W["k_idx"] = W["k_idx"].copy()
        W["k_idx"][b, j, 3] = 0x7F if kdt == E4M3 else 0x7FC0  # NaN
        _, _, _, st = gc.gpu_select_attend(W)
        assert st == want, (b, j)
