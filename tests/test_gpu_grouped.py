"""GPU parity of the grouped candidate sets ("PaperTrace 2.2 · Fine-grained indexing", §2
eq. (5)): G groups of query heads, each with the selection of its own index heads.

Per group the selection is checked like the shared one (a valid top-k of the oracle's fp64
scores of the group's index heads, within twice the score tolerance, exactly the oracle's
set where the cutoff is separated), and the group's query heads against the oracle's
attention over the GPU's candidates.  G = 1 must equal the shared fused call bit for bit.
"""
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


def _say(x):
    print(x, flush=True)


def gpu_grouped(W, G):
    P, d = device_workload(W)
    O, lse, _ = empty_outputs(W, gc.out_dtype(W))
    idx = torch.full((G, W["B"], W["n_q"], W["k"]), -7, dtype=torch.int32, device="cuda")
    ws = sa.grouped_workspace(P, G)
    sa.sa_select_attend_grouped(P, G, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse, ws)
    st = sa.sa_device_status(ws)
    return idx.cpu().numpy(), O.float().cpu().numpy(), lse.cpu().numpy(), st


def check_grouped(W, G, rows):
    idx, O, lse, st = gpu_grouped(W, G)
    assert st == sa.SA_OK
    exact = 0
    Hg = W["Hq"] // G
    for g in range(G):
        Wg = orc.group_workload(W, G, g)
        sc = orc.scores(Wg, rows)
        ref_idx, sk, _, _ = orc.select(Wg, sc, rows)
        gi = idx[g].reshape(-1, W["k"])[rows]
        r = check_index_rows(Wg, rows, gi, sc, ref_idx, sk)
        exact += r["exact_rows"]
        O_or, lse_or = orc.attend(Wg, gi, rows)
        gc.compare_attention(Wg, rows, O[:, g * Hg:(g + 1) * Hg], lse[:, g * Hg:(g + 1) * Hg], O_or, lse_or)
    return idx, exact


CASES = {
    "mha_bf16_ragged_g2": (dict(seed=51, B=2, n_q=200, n_kv=200, Hq=4, Hkv=4, d_qk=128, d_v=128, Hidx=16, d_idx=64,
                                k=32, lens=[200, 151]), 2),
    "mha_bf16_ragged_g4": (dict(seed=51, B=2, n_q=200, n_kv=200, Hq=4, Hkv=4, d_qk=128, d_v=128, Hidx=16, d_idx=64,
                                k=32, lens=[200, 151]), 4),
    "c1_n512_g2": (dict(cid=1, n=512), 2),
    "c3_b8_kv3000_k256_g2": (dict(cid=3, B=8, n_kv=3000, k=256), 2),
    "c3_b8_kv3000_k256_g4": (dict(cid=3, B=8, n_kv=3000, k=256), 4),
    "c2_n1000_k256_g2": (dict(cid=2, n=1000, k=256), 2),
}


def _workload(name):
    kw, G = CASES[name]
    if "cid" in kw:
        return gc.workload(name.rsplit("_g", 1)[0], **kw), G
    return sa_synth.custom(**kw), G


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_sets_against_the_oracle(name):
    W, G = _workload(name)
    _say("grouped %s" % name)
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    idx, exact = check_grouped(W, G, rows)
    _say("grouped %s: exact rows %d of %d" % (name, exact, G * rows.size))
    if G > 1 and W["n_kv"] > 2 * W["k"]:  # the groups' index heads differ, so (with k well below
        # the history) their sets differ
        assert not np.array_equal(idx[0], idx[1])


@pytest.mark.parametrize("name", ["mha_bf16_ragged_g2", "c3_b8_kv3000_k256_g2"])
def test_one_group_equals_the_shared_call(name):
    W, _ = _workload(name)
    idx1, O1, lse1, st1 = gpu_grouped(W, 1)
    idx, O, lse, st = gc.gpu_select_attend(W)
    assert st1 == sa.SA_OK and st == sa.SA_OK
    assert np.array_equal(idx1[0], idx) and np.array_equal(O1, O) and np.array_equal(lse1, lse)


def test_full_size_bf16_prefill_two_groups():
    _say("grouped full c1: generate")
    W = sa_synth.make_config(1)
    rows = gc.sample_rows(W, n_each=8, n_rand=40)
    _say("grouped full c1: %d rows" % rows.size)
    check_grouped(W, 2, rows)
