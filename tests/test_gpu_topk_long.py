"""Top-k over long rows (more than 8192 visible positions): many rows (one workgroup per row,
row in registers) and few rows (a histogram over slices, then one workgroup per row that
streams the row).  The selection of given fp32 scores must equal the oracle's select bit for
bit, including the lower-position rule for exact ties at the cutoff.  Score patterns: Gaussian, a narrow band
(every key in a few top-level bins), a cutoff tie group too large for the candidate list
(the register fallback), all-equal rows, signed values with +-0, and causal rows whose
lengths are not multiples of the chunk width."""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


def _scores(kind, n_rows, n_kv, seed):
    rng = np.random.default_rng(seed)
    if kind == "gauss":
        s = rng.standard_normal((n_rows, n_kv))
    elif kind == "narrow":
        s = 100.0 + 0.01 * rng.standard_normal((n_rows, n_kv))
    elif kind in ("big_tie_bin", "huge_tie_bin"):
        s = rng.random((n_rows, n_kv))
        nt = 6000 if kind == "big_tie_bin" else 12000
        for r in range(n_rows):
            pos = rng.permutation(n_kv)
            s[r, pos[:1000]] = 100.0 + rng.random(1000)
            s[r, pos[1000:1000 + nt]] = 5.0  # the cutoff falls inside nt exact ties
    elif kind == "all_equal":
        s = np.full((n_rows, n_kv), 0.25)
    elif kind == "signed_zeros":
        s = rng.standard_normal((n_rows, n_kv))
        s[:, ::7] = 0.0
        s[:, 3::7] = -0.0
        s[:, 5::11] = -1e-30
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


@pytest.mark.parametrize("kind,n_kv,causal,n_q", [
    ("gauss", 20000, 0, 520), ("narrow", 20000, 0, 520), ("big_tie_bin", 20000, 0, 520),
    ("all_equal", 12000, 0, 520), ("signed_zeros", 12000, 0, 520), ("gauss", 30001, 1, 520),
    ("big_tie_bin", 16385, 1, 520),
    # 512 rows or fewer: histogram over slices, one streaming workgroup per row
    ("gauss", 70000, 0, 8), ("narrow", 65536, 1, 8), ("big_tie_bin", 40000, 0, 8),
    ("huge_tie_bin", 40000, 0, 8), ("all_equal", 20000, 0, 4), ("signed_zeros", 9000, 0, 4),
    ("gauss", 200003, 0, 3),
])
def test_long_row_topk_matches_oracle(kind, n_kv, causal, n_q):
    k = 2048
    q_pos0 = [n_kv - n_q] if causal else None
    W = sa_synth.custom(B=1, n_q=n_q, n_kv=n_kv, k=k, causal=causal, q_pos0=q_pos0, with_main=False)
    print("topk long %s n_kv=%d causal=%d n_q=%d" % (kind, n_kv, causal, n_q), flush=True)
    s = _scores(kind, n_q, n_kv, seed=n_kv + causal)
    sc = torch.from_numpy(s.reshape(1, n_q, n_kv)).cuda()
    idx, vals, st = gc.gpu_topk(W, sc)
    assert st == sa.SA_OK
    rows = np.arange(n_q, dtype=np.int32)
    sc64 = s.astype(np.float64)
    ref_idx, *_ = orc.select(W, sc64, rows)
    got = idx.reshape(ref_idx.shape)
    bad = np.nonzero((got != ref_idx).any(axis=1))[0]
    assert bad.size == 0, ("rows differ", bad[:5].tolist())
    v = vals.reshape(ref_idx.shape)
    want = np.where(ref_idx >= 0, sc64[rows[:, None], np.maximum(ref_idx, 0)], -np.inf).astype(np.float32)
    assert np.array_equal(v.view(np.uint32), want.view(np.uint32)) or np.array_equal(v, want)
