"""The environment switches of the library on the GPU.

SA_DEBUG_CHECKS=1: a check kernel reads every candidate list before the attention and sets
SA_ERR_INDEX when a list repeats a position (duplicates must be removed before the softmax:
"PaperTrace 2.2 · Fine-grained indexing", §2.1; "PaperTrace 2.1.1 · Hashing and
clustering", §5.1) or holds an entry that is neither -1 nor visible.  The library's own
selections never trip it.  SA_FORCE_UNFUSED=1 selects through stored score rows instead of
the streaming selection (same result, bit for bit); SA_SPLITS overrides the split count of
the latent attention (same softmax up to the merge's rounding)."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from tests.device_inputs import empty_outputs
from token_selector_gather_amd.inputs import device_workload

pytestmark = pytest.mark.gpu
E4M3 = sa_synth.E4M3


def _say(x):
    print(x, flush=True)


def _attn_status(W, idx_np, paged=False):
    P, d = device_workload(W)
    O, lse, _ = empty_outputs(W, gc.out_dtype(W))
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    ws = sa.workspace(P, sa.SA_OP_SPARSE_ATTN)
    sa.sa_sparse_attn(P, d["Q"], d["K"], d["V"], idx, O, lse, ws)
    return sa.sa_device_status(ws)


def _clean_lists(W, seed=0):
    """Ascending, distinct, visible candidates per row (-1 padded), from the oracle's selection."""
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    idx, *_ = orc.select(W, orc.scores(W, rows), rows)
    return idx.reshape(W["B"], W["n_q"], W["k"])


@pytest.mark.parametrize("latent", [False, True])
def test_debug_checks_flag_repeats_and_invisible_entries(latent, monkeypatch):
    if latent:
        W = sa_synth.custom(seed=61, B=2, n_q=1, n_kv=700, Hq=64, Hkv=1, d_qk=576, d_v=512, mla=True, Hidx=8,
                            d_idx=64, kidx_dtype=E4M3, k=128, lens=[700, 300], q_pos0=[699, 299])
    else:
        W = sa_synth.custom(seed=62, B=2, n_q=96, n_kv=300, Hq=4, Hkv=2, d_qk=64, d_v=64, Hidx=4, d_idx=32, k=24,
                            lens=[300, 200])
    idx = _clean_lists(W)
    monkeypatch.setenv("SA_DEBUG_CHECKS", "1")
    assert _attn_status(W, idx) == sa.SA_OK
    # a repeated visible position in one row
    dup = idx.copy()
    b, i = W["B"] - 1, W["n_q"] - 1
    dup[b, i, 1] = dup[b, i, 0]
    assert _attn_status(W, dup) == sa.SA_ERR_INDEX
    # a position past the row's visible prefix
    inv = idx.copy()
    Ls = [min(int(W["q_pos0"][bb]) + 1, int(W["kv_len"][bb])) for bb in range(W["B"])]  # row 0 of each batch
    bb = int(np.argmin(Ls))
    assert Ls[bb] < W["n_kv"]
    inv[bb, 0, 0] = Ls[bb]
    assert _attn_status(W, inv) == sa.SA_ERR_INDEX
    # a negative entry other than -1
    neg = idx.copy()
    neg[0, 0, 2] = -5
    assert _attn_status(W, neg) == sa.SA_ERR_INDEX
    # without the switch the same lists run and report nothing
    monkeypatch.delenv("SA_DEBUG_CHECKS")
    assert _attn_status(W, dup) == sa.SA_OK


def test_debug_checks_pass_the_library_selection(monkeypatch):
    monkeypatch.setenv("SA_DEBUG_CHECKS", "1")
    for cid in (0, 1):
        W = sa_synth.make_config(cid, n=512) if cid == 1 else sa_synth.make_config(cid)
        _, _, _, st = gc.gpu_select_attend(W)
        assert st == sa.SA_OK, cid


def test_force_unfused_gives_the_streaming_selection(monkeypatch):
    W = sa_synth.custom(seed=63, B=2, n_q=2048, n_kv=2048, Hq=2, Hkv=2, d_qk=64, d_v=64, Hidx=64, d_idx=128,
                        kidx_dtype=E4M3, k=100, lens=[2048, 1500], with_main=False)
    P, d = device_workload(W, with_main=False)

    def run():
        ws = sa.workspace(P, sa.SA_OP_SELECT)
        idx = torch.full((W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
        sa.sa_select(P, d["q_idx"], d["k_idx"], d["w"], idx, ws)
        assert sa.sa_device_status(ws) == sa.SA_OK
        return idx.cpu().numpy()

    fused = run()
    monkeypatch.setenv("SA_FORCE_UNFUSED", "1")
    unfused = run()
    np.testing.assert_array_equal(fused, unfused)


def test_splits_override_keeps_the_latent_attention(monkeypatch):
    W = sa_synth.custom(seed=64, B=3, n_q=1, n_kv=5000, Hq=128, Hkv=1, d_qk=576, d_v=512, mla=True, Hidx=8,
                        d_idx=64, kidx_dtype=E4M3, k=512, lens=[5000, 2000, 100], q_pos0=[4999, 1999, 99])
    idx = _clean_lists(W)
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    O_or, lse_or = orc.attend(W, idx.reshape(len(rows), -1), rows)
    for s in ("1", "3", "16"):
        monkeypatch.setenv("SA_SPLITS", s)
        O, lse = gc.gpu_sparse_attn(W, idx)
        err_o, err_l = gc.compare_attention(W, rows, O, lse, O_or, lse_or)
        _say("SA_SPLITS=%s: max|dO| %.3g max|dLSE| %.3g" % (s, err_o, err_l))


def test_bf16_split_partials_cost_about_one_rounding(monkeypatch):
    """The latent attention stores each split's o / l in bf16 before the log-sum-exp merge
    (block-mixture identity, COBS reading note eq. (P3)).  That is one extra rounding of a
    value of the output's own size: against the unsplit run (no partials) every output stays
    within two bf16 steps of its (row, head)'s largest value, and the error against the oracle
    does not grow beyond that."""
    W = sa_synth.custom(seed=65, B=4, n_q=1, n_kv=6000, Hq=128, Hkv=1, d_qk=576, d_v=512, mla=True, Hidx=8,
                        d_idx=64, kidx_dtype=E4M3, k=2048, lens=[6000, 4100, 2500, 2048],
                        q_pos0=[5999, 4099, 2499, 2047])
    idx = _clean_lists(W)
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    O_or, lse_or = orc.attend(W, idx.reshape(len(rows), -1), rows)
    monkeypatch.setenv("SA_SPLITS", "1")
    O1, lse1 = gc.gpu_sparse_attn(W, idx)
    e1, _ = gc.compare_attention(W, rows, O1, lse1, O_or, lse_or)
    scale = np.abs(O1).max(axis=-1, keepdims=True)  # per (batch, head, row)
    for s in ("4", "16"):
        monkeypatch.setenv("SA_SPLITS", s)
        Os, lses = gc.gpu_sparse_attn(W, idx)
        es, _ = gc.compare_attention(W, rows, Os, lses, O_or, lse_or)
        steps = np.abs(Os - O1) / (scale * 2.0 ** -8)  # in bf16 steps of the largest value
        _say("SA_SPLITS=%s: max|O_split - O_unsplit| = %.2f bf16 steps of the row's largest value; "
             "max|dO| vs oracle %.3g (unsplit %.3g)" % (s, steps.max(), es, e1))
        assert steps.max() <= 2.0
        assert es <= e1 + 2.0 ** -7 * scale.max()
        np.testing.assert_allclose(lses, lse1, rtol=0, atol=1e-5 * max(1.0, np.abs(lse1).max()))
