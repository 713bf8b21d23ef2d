"""GPU parity of the indexer's many-row prefill layout (one pass over the history per block
of query rows, keys widened to bf16 once per chunk), which serves workloads with thousands
of query rows.  Sampled rows of the standalone score call (NaN-preserving ReLU, invisible
entries filled) and of the fused call (finite inputs, plain ReLU) against the oracle
("PaperTrace 2.2 · Fine-grained indexing", §2.1 eq. (1); the score definition of the
Lightning indexer)."""
import numpy as np
import pytest

import sa_synth
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
