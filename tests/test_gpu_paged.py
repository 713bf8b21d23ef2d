"""GPU parity of the paged sparse attention (sa_sparse_attn_paged).

"PaperTrace 2.2 · Fine-grained indexing", §2.1 (the main-KV gather goes through the block
table to physical rows) and §3.1 (block_table among the objects of the attention call).
Paging is a storage layout, so the paged call must reproduce the contiguous call bit for
bit on the same candidates (same kernels, same arithmetic order), and both must match the
oracle; the pools are filled by a seeded random page permutation with poisoned spare rows.
"""
import numpy as np
import pytest
import torch

import sa_synth
import token_selector_gather_amd as sa
from oracle import oracle as orc
from tests import gpu_common as gc
from token_selector_gather_amd.inputs import device_workload
from tests.device_inputs import device_pool, empty_outputs

pytestmark = pytest.mark.gpu


def _say(x):
    print(x, flush=True)


def _run_both(W, idx_np, ps, bt=None, pool_rows=None, spare=3, call_bt=None, fill=3.0e4):
    """(contiguous O, lse), (paged O, lse) on the same candidates; returns numpy arrays.
    The pool is filled along bt, its unused rows with `fill`; the paged call reads through
    call_bt (default bt)."""
    P, d = device_workload(W)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32).reshape(W["B"], W["n_q"], -1)).cuda()
    ws = sa.workspace(P, sa.SA_OP_SPARSE_ATTN)
    wsp = sa.workspace(P, sa.SA_OP_SPARSE_ATTN_PAGED)
    O1, l1, _ = empty_outputs(W, gc.out_dtype(W))
    sa.sa_sparse_attn(P, d["Q"], d["K"], d["V"], idx, O1, l1, ws)
    if bt is None:
        bt, pool_rows = sa_synth.paged_layout(W["seed"] + 7, W["B"], W["n_kv"], ps, spare)
    Kp = device_pool(d["K"], bt, ps, pool_rows, fill)
    latent = W.get("V") is None
    Vp = Kp[..., : W["d_v"]] if latent else device_pool(d["V"], bt, ps, pool_rows, fill)
    btd = torch.from_numpy(np.ascontiguousarray(bt if call_bt is None else call_bt, dtype=np.int32)).cuda()
    O2, l2, _ = empty_outputs(W, gc.out_dtype(W))
    sa.sa_sparse_attn_paged(P, d["Q"], Kp, Vp, btd, ps, idx, O2, l2, wsp)
    torch.cuda.synchronize()
    return ((O1.float().cpu().numpy(), l1.cpu().numpy()), (O2.float().cpu().numpy(), l2.cpu().numpy()))


def _same(a, b):
    assert np.array_equal(a[0], b[0]), "O differs between paged and contiguous"
    assert np.array_equal(a[1], b[1]), "LSE differs between paged and contiguous"


CASES = {
    "mha_bf16_ragged_p16": (dict(seed=31, B=2, n_q=300, n_kv=300, Hq=2, Hkv=2, d_qk=128, d_v=128, k=32,
                                 lens=[300, 211]), 16),
    "mha_bf16_d64_p1": (dict(seed=32, B=1, n_q=96, n_kv=200, Hq=3, Hkv=3, d_qk=64, d_v=64, k=40, q_pos0=[104],
                             causal=1), 1),
    "mha_bf16_d256_noncausal_p256": (dict(seed=33, B=2, n_q=8, n_kv=700, Hq=2, Hkv=2, d_qk=256, d_v=256, k=64,
                                          causal=0), 256),
}
LATENT = {
    "c3_b8_kv3000_k256_p64": (dict(cid=3, B=8, n_kv=3000, k=256), 64),
    "c2_n1000_k256_p64": (dict(cid=2, n=1000, k=256), 64),
    "c4_kv5000_k128_p32": (dict(cid=4, n_kv=5000, k=128), 32),
}


def _workload(name):
    if name in CASES:
        kw, ps = CASES[name]
        kw = dict(kw)
        if "q_pos0" in kw:
            kw["q_pos0"] = np.asarray(kw["q_pos0"], np.int32)
        return sa_synth.custom(**kw), ps
    kw, ps = LATENT[name]
    return gc.workload(name, **kw), ps


@pytest.mark.parametrize("name", list(CASES) + list(LATENT))
def test_paged_equals_contiguous_and_oracle(name):
    W, ps = _workload(name)
    _say("paged %s: select" % name)
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    ref = orc.select_attend(W, rows)
    _say("paged %s: attend" % name)
    a, b = _run_both(W, ref["idx"], ps)
    _same(a, b)
    gc.compare_attention(W, rows, b[0], b[1], ref["O"], ref["lse"])


def test_paged_mha_against_the_oracle_on_the_host_pool():
    # the oracle's own paged path on the same pool layout the device pool is built from
    W, ps = _workload("mha_bf16_ragged_p16")
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    ref = orc.select_attend(W, rows)
    bt, pool_rows = sa_synth.paged_layout(W["seed"] + 7, W["B"], W["n_kv"], ps, 3)
    fill = sa_synth.encode(np.array([3.0e4]), W["main_dtype"])[0]
    O_or, l_or = orc.attend_paged(W, ref["idx"], sa_synth.to_pool(W["K"], bt, ps, pool_rows, fill),
                                  sa_synth.to_pool(W["V"], bt, ps, pool_rows, fill), bt, ps, rows)
    _, b = _run_both(W, ref["idx"], ps, bt, pool_rows)
    gc.compare_attention(W, rows, b[0], b[1], O_or, l_or)


@pytest.mark.parametrize("name", ["mha_bf16_ragged_p16", "c3_b8_kv3000_k256_p64"])
def test_pages_outside_the_pool_skip_their_candidates(name):
    W, ps = _workload(name)
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    ref = orc.select_attend(W, rows)
    bt, pool_rows = sa_synth.paged_layout(W["seed"] + 7, W["B"], W["n_kv"], ps, 3)
    bad = bt.copy()
    bad[0, 1] = -5
    bad[-1, 0] = pool_rows // ps  # one past the last pool page
    idx = ref["idx"].reshape(W["B"], W["n_q"], -1)
    drop = idx.copy()
    page = np.where(drop >= 0, drop // ps, -1)
    drop[0][page[0] == 1] = -1
    drop[-1][page[-1] == 0] = -1
    _, b = _run_both(W, idx, ps, bt, pool_rows, call_bt=bad)
    a, _ = _run_both(W, drop, ps, bt, pool_rows)
    _same(a, b)
    O_or, l_or = orc.attend(W, drop.reshape(len(rows), -1), rows)
    gc.compare_attention(W, rows, b[0], b[1], O_or, l_or)


@pytest.mark.parametrize("cid,ps", [(1, 64), (3, 64)])
def test_full_size_paged_equals_contiguous(cid, ps):
    # at full size, on the selection the fused call makes (the benchmark's configuration)
    _say("paged full c%d: generate" % cid)
    W = sa_synth.make_config(cid)
    idx, O, lse, st = gc.gpu_select_attend(W)
    assert st == sa.SA_OK
    _say("paged full c%d: attend" % cid)
    a, b = _run_both(W, idx, ps)
    _same(a, b)
    Og, Lg = O, lse
    assert np.array_equal(b[0], Og) and np.array_equal(b[1], Lg)
    rows = gc.sample_rows(W, n_each=4, n_rand=12)
    O_or, l_or = orc.attend(W, idx.reshape(W["B"] * W["n_q"], -1)[rows], rows)
    gc.compare_attention(W, rows, b[0], b[1], O_or, l_or)


@pytest.mark.parametrize("name,ps", [("mha_bf16_ragged_p16", 16), ("mha_bf16_ragged_p16", 64),
                                     ("c3_b8_kv3000_k256_p64", 64)])
def test_nan_in_rows_no_entry_selects_never_reaches_the_outputs(name, ps):
    # K/V rows past kv_len (kv_len not a multiple of 64), visible rows that no query row of
    # the batch selected, and the pool's unused rows all hold bf16 NaN: neither the
    # contiguous nor the paged call may let them into an output.  The multi-head shape runs
    # the tile kernel (whole 64-key tiles per block of 64 query rows), the latent one the
    # gather kernel.
    W, _ = _workload(name)
    rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    ref = orc.select_attend(W, rows)
    idx = ref["idx"].reshape(W["B"], W["n_q"], -1)
    Wn = W.__class__(W)
    keys = ("K",) if W.get("V") is None else ("K", "V")
    for key in keys:
        Wn[key] = W[key].copy()
    n_poison = 0
    for b in range(W["B"]):
        used = np.zeros(W["n_kv"], bool)
        sel = idx[b][idx[b] >= 0]
        used[sel] = True
        used[int(W["kv_len"][b]):] = False
        poison = np.where(~used)[0]
        assert int(W["kv_len"][b]) % 64 != 0 or b > 0
        n_poison += poison.size
        for key in keys:
            Wn[key][b][:, poison, :] = 0x7FC0
    _say("nan rows %s p%d: %d poisoned rows" % (name, ps, n_poison))
    assert n_poison > 0
    a, b2 = _run_both(Wn, idx, ps, fill=float("nan"))
    _same(a, b2)
    gc.compare_attention(W, rows, a[0], a[1], ref["O"], ref["lse"])
