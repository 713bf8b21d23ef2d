"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark
times (sa_select_attend), on stratified row samples the oracle can score one by one.

The planted-needle decode additionally checks needle recall (16 of 16 per query, GPU and
oracle) and the exact-tie groups planted at each query's cutoff ("PaperTrace 2.2 ·
Fine-grained indexing", §2.1 and §3.1: ties resolve to the lower positions).
"""
import numpy as np
import pytest

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from tests.c4_plant import plant_cutoff_ties
from tests.checker import check_index_rows, tie_groups_of

pytestmark = pytest.mark.gpu


def _say(x):
    print(x, flush=True)


def test_full_c1_bf16_prefill():
    _say("full c1: generate")
    W = sa_synth.make_config(1)
    rows = gc.sample_rows(W, n_each=24, n_rand=80)
    _say("full c1: %d rows" % rows.size)
    r = gc.full_check(W, rows=rows)
    _say("full c1: exact rows %d band rows %d |dO| %.3g" % (r["exact_rows"], r["band_rows"], r["err_o"]))


def test_full_c2_mla_prefill():
    # the stratified sample: the first 64 and last 64 query rows and 384 random ones
    _say("full c2: generate")
    W = sa_synth.make_config(2)
    rows = gc.stratified_rows(W, 64, 64, 384)
    assert rows.size == 512
    _say("full c2: %d rows" % rows.size)
    r = gc.full_check(W, rows=rows, check_sparse=True, say=lambda x: _say("full c2: " + x))
    _say("full c2: exact rows %d band rows %d |dO| %.3g (bound 2e-2), on the oracle's sets %.3g"
         % (r["exact_rows"], r["band_rows"], r["err_o"], r["err_o_sparse"]))


def test_full_c3_mla_decode():
    _say("full c3: generate")
    W = sa_synth.make_config(3)
    r = gc.full_check(W)
    _say("full c3: exact rows %d band rows %d |dO| %.3g" % (r["exact_rows"], r["band_rows"], r["err_o"]))


def test_full_c4_needles_and_cutoff_ties():
    _say("full c4: generate and plant ties")
    W = plant_cutoff_ties(sa_synth.make_config(4))
    rows = np.arange(W["n_q"], dtype=np.int32)
    sc = orc.scores(W, rows)
    planted = W["tie_groups_planted"]
    assert len(planted) == W["n_q"], sorted(planted)
    # needles: each query's 16 needles score at least 3 standard deviations above every other key
    for i in rows:
        npos = W["needle_pos"][0, i]
        rest = np.delete(sc[i], npos)
        assert sc[i][npos].min() >= rest.max() + 3 * rest.std(), i
    groups = {0: tie_groups_of(W["k_idx"][0], int(W["kv_len"][0]))}
    r = gc.full_check(W, rows=rows, tie_groups=groups)
    idx = r["idx"].reshape(W["n_q"], -1)
    ref_idx = r["ref_idx"]
    for i in rows:
        npos = set(W["needle_pos"][0, i].tolist())
        assert npos <= set(idx[i].tolist()), ("GPU needle recall", i)
        assert npos <= set(ref_idx[i].tolist()), ("oracle needle recall", i)
    # every planted group straddles its query's cutoff and its selected members are its lowest positions
    for row, grp in planted.items():
        chosen = [j for j in grp if j in set(idx[row].tolist())]
        assert 0 < len(chosen) < len(grp), (row, grp, chosen)
        assert chosen == grp[: len(chosen)]
    _say("full c4: %d tie groups, exact rows %d band rows %d" % (len(planted), r["exact_rows"], r["band_rows"]))
