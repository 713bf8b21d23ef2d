"""CPU-only checks of the C ABI: the library loads, exports every function include/sa.h
declares, and rejects malformed arguments synchronously (before any launch, so no GPU
is touched).  Device pointers here are fake aligned addresses that are never dereferenced."""
import ctypes
import os
import re

import pytest

import token_selector_gather_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")

needs_lib = pytest.mark.skipif(not os.path.exists(sa.LIB_PATH), reason="libsa.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for f in ("sa_indexer_score", "sa_topk", "sa_sparse_attn", "sa_select_attend", "sa_workspace_bytes",
              "sa_device_status", "sa_status_str", "sa_abi_version"):
        assert f in names


@needs_lib
def test_library_exports_every_declared_function():
    L = ctypes.CDLL(sa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


@needs_lib
def test_abi_version_and_status_strings():
    assert sa.sa_abi_version() == sa.ABI_VERSION
    assert sa.sa_status_str(sa.SA_OK) == "SA_OK"
    assert sa.sa_status_str(sa.SA_ERR_NONFINITE) == "SA_ERR_NONFINITE"
    assert sa.sa_status_str(sa.SA_ERR_INDEX) == "SA_ERR_INDEX"
    assert sa.sa_status_str(99) == "SA_ERR_UNKNOWN"


FAKE = 0x10000  # 256-byte aligned, never dereferenced on the error paths below


def _prob(**kw):
    base = dict(B=2, n_q=64, n_kv=64, Hq=4, Hkv=4, d_qk=64, d_v=64, Hidx=4, d_idx=32, k=8, causal=1)
    base.update(kw)
    return sa._Problem(*[base[f] for f in sa.Problem.FIELDS], None, None, 0.0)


def _t(dtype=sa.SA_BF16, s0=64 * 64 * 4, s1=64 * 64, s2=64, data=FAKE):
    return sa._Tensor(data, dtype, s0, s1, s2)


@needs_lib
@pytest.mark.parametrize("field,value", [("B", 0), ("n_q", 0), ("n_kv", -1), ("k", 0), ("Hq", 3), ("Hkv", 0),
                                         ("causal", 2), ("d_idx", 0)])
def test_malformed_problem_is_rejected(field, value):
    L = sa.lib()
    p = _prob(**{field: value})
    assert L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SELECT_ATTEND) == 0
    rc = L.sa_topk(ctypes.byref(p), FAKE, 64, FAKE, None, FAKE, 1 << 20, None)
    assert rc == sa.SA_ERR_INVALID_ARG


@needs_lib
def test_workspace_errors():
    L = sa.lib()
    p = _prob()
    need = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_TOPK)
    assert need >= 256
    assert L.sa_topk(ctypes.byref(p), FAKE, 64, FAKE, None, None, need, None) == sa.SA_ERR_WORKSPACE
    assert L.sa_topk(ctypes.byref(p), FAKE, 64, FAKE, None, FAKE, need - 1, None) == sa.SA_ERR_WORKSPACE
    assert L.sa_topk(ctypes.byref(p), FAKE, 64, FAKE, None, FAKE + 16, need, None) == sa.SA_ERR_WORKSPACE
    assert L.sa_topk(ctypes.byref(p), FAKE, 63, FAKE, None, FAKE, need, None) == sa.SA_ERR_INVALID_ARG
    sel = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SELECT_ATTEND)
    assert sel >= 256 + 2 * 64 * 64 * 4 + 2 * 64 * 8 * 4  # status + score rows + selection (small: two-pass)


@needs_lib
def test_streaming_selection_workspace_holds_no_score_matrix():
    # the latent prefill (n = 32768, 64 x 128 index heads, k = 2048): the fused call's
    # workspace holds candidate lists of the rows in flight, not B n_q n_kv scores
    L = sa.lib()
    p = sa._Problem(1, 32768, 32768, 128, 1, 576, 512, 64, 128, 2048, 1, None, None, 0.0)
    scores = 32768 * 32768 * 4
    for op in (sa.SA_OP_SELECT, sa.SA_OP_SELECT_ATTEND):
        need = L.sa_workspace_bytes(ctypes.byref(p), op)
        assert 0 < need < scores // 4, (op, need)  # candidate lists (+ the selection buffer), not scores
    # a small problem keeps the stored scores (the two-pass selection)
    q = _prob()
    assert L.sa_workspace_bytes(ctypes.byref(q), sa.SA_OP_SELECT) >= 256 + 2 * 64 * 64 * 4
    # the active-head selections at that size score their (16) heads through the same
    # streaming selection: no score rows either (with 16 heads a block holds 64 query rows,
    # so four times the rows are in flight)
    for g in (8, 16):
        assert 0 < L.sa_misa_workspace_bytes(ctypes.byref(p), 128, g) < scores // 2
    assert 0 < L.sa_resmisa_workspace_bytes(ctypes.byref(p), 128, 10) < scores // 2


@needs_lib
def test_select_argument_errors():
    L = sa.lib()
    p = _prob()
    need = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SELECT)
    q, k, w = _t(s0=64 * 4 * 32, s1=4 * 32, s2=32), _t(s0=64 * 32, s1=32, s2=0), _t(dtype=sa.SA_F32, s0=64 * 4, s1=4, s2=0)
    call = lambda idx=FAKE, ws=FAKE, n=need, qq=q: L.sa_select(ctypes.byref(p), qq, k, w, idx, ws, n, None)
    assert call(idx=None) == sa.SA_ERR_INVALID_ARG
    assert call(idx=FAKE + 2) == sa.SA_ERR_INVALID_ARG
    assert call(ws=None) == sa.SA_ERR_WORKSPACE
    assert call(n=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(qq=_t(dtype=sa.SA_FP8_E4M3, s0=64 * 4 * 32, s1=4 * 32, s2=32)) == sa.SA_ERR_UNSUPPORTED


@needs_lib
def test_no_alloc_argument_errors():
    # checked on the host before the library looks for its scratch or launches anything
    L = sa.lib()
    q, k, w = _t(s0=64 * 4 * 32, s1=4 * 32, s2=32), _t(s0=64 * 32, s1=32, s2=0), _t(dtype=sa.SA_F32, s0=64 * 4, s1=4, s2=0)
    ok = _t()
    call = lambda pp, status=None, idx=FAKE: L.sa_select_attend_noalloc(ctypes.byref(pp), q, k, w, ok, ok, ok, idx, ok,
                                                                         None, status, None)
    assert call(_prob(), status=FAKE + 16) == sa.SA_ERR_INVALID_ARG  # status word not 256-byte aligned
    assert call(_prob(), idx=FAKE + 2) == sa.SA_ERR_INVALID_ARG
    assert call(_prob(k=0)) == sa.SA_ERR_INVALID_ARG
    big = _prob(n_q=4096, n_kv=4096, k=64)  # scores of 64 MiB plus the rest: beyond the fixed scratch
    assert L.sa_workspace_bytes(ctypes.byref(big), sa.SA_OP_SELECT_ATTEND) > 64 << 20
    assert call(big) == sa.SA_ERR_WORKSPACE


@needs_lib
def test_attention_argument_errors():
    L = sa.lib()
    p = _prob()
    ws = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SPARSE_ATTN)
    ok = _t()
    call = lambda Q=ok, K=ok, V=ok, O=ok, idx=FAKE, lse=None, pp=p: L.sa_sparse_attn(
        ctypes.byref(pp), Q, K, V, idx, O, lse, FAKE, ws, None)
    assert call(idx=None) == sa.SA_ERR_INVALID_ARG
    assert call(Q=_t(data=None)) == sa.SA_ERR_INVALID_ARG
    assert call(K=_t(data=FAKE + 2)) == sa.SA_ERR_INVALID_ARG          # misaligned
    assert call(V=_t(s2=60)) == sa.SA_ERR_INVALID_ARG                  # stride not 16-byte multiple
    assert call(O=_t(dtype=sa.SA_F32)) == sa.SA_ERR_UNSUPPORTED        # mixed dtypes
    assert call(Q=_t(dtype=7), K=_t(dtype=7), V=_t(dtype=7), O=_t(dtype=7)) == sa.SA_ERR_UNSUPPORTED
    assert call(lse=FAKE + 1) == sa.SA_ERR_INVALID_ARG
    odd = _prob(d_qk=48, d_v=48)  # lanes per row not a power of two
    assert call(pp=odd) == sa.SA_ERR_UNSUPPORTED
    gqa3 = _prob(Hq=12, Hkv=4)  # group of 3 query heads per key/value head
    assert call(pp=gqa3) == sa.SA_ERR_UNSUPPORTED


@needs_lib
def test_paged_attention_argument_errors():
    L = sa.lib()
    p = _prob()
    ws = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SPARSE_ATTN_PAGED)
    assert ws >= 256 + 2 * 64 * 8 * 4  # status + translated candidate rows
    ok = _t(s0=0)

    def call(pool_rows=4096, bt=FAKE, bt_stride=4, page=16, pp=p, K=ok, Q=ok):
        return L.sa_sparse_attn_paged(ctypes.byref(pp), Q, K, ok, pool_rows, bt, bt_stride, page, FAKE, ok,
                                      None, FAKE, ws, None)
    assert call(bt=None) == sa.SA_ERR_INVALID_ARG
    assert call(bt=FAKE + 2) == sa.SA_ERR_INVALID_ARG
    assert call(page=24) == sa.SA_ERR_INVALID_ARG       # not a power of two
    assert call(page=0) == sa.SA_ERR_INVALID_ARG
    assert call(page=1 << 17) == sa.SA_ERR_INVALID_ARG
    assert call(bt_stride=3) == sa.SA_ERR_INVALID_ARG   # 64 positions need 4 pages of 16
    assert call(pool_rows=0) == sa.SA_ERR_INVALID_ARG
    assert call(K=_t(s0=0, data=FAKE + 2)) == sa.SA_ERR_INVALID_ARG
    f32 = _t(dtype=sa.SA_F32, s0=0)
    assert L.sa_sparse_attn_paged(ctypes.byref(p), f32, f32, f32, 4096, FAKE, 4, 16, FAKE, f32, None, FAKE, ws,
                                  None) == sa.SA_ERR_UNSUPPORTED  # only the bf16 kernels translate pages
    gqa = _prob(Hq=8, Hkv=4)
    ws2 = L.sa_workspace_bytes(ctypes.byref(gqa), sa.SA_OP_SPARSE_ATTN_PAGED)
    assert L.sa_sparse_attn_paged(ctypes.byref(gqa), ok, ok, ok, 4096, FAKE, 4, 16, FAKE, ok, None, FAKE, ws2,
                                  None) == sa.SA_ERR_UNSUPPORTED
    assert call(pool_rows=1 << 24) == sa.SA_ERR_UNSUPPORTED  # 24-bit row products of the MHA kernel
    big = _prob(k=6)
    assert call(pp=big) == sa.SA_ERR_UNSUPPORTED             # MHA kernel reads candidates four at a time


@needs_lib
def test_grouped_selection_argument_errors():
    L = sa.lib()
    p = _prob(Hidx=8)
    wsz = lambda pp, g: L.sa_grouped_workspace_bytes(ctypes.byref(pp), g)
    assert wsz(p, 2) > 256 and wsz(p, 1) > 256
    assert wsz(p, 0) == 0                    # no groups
    assert wsz(p, 3) == 0                    # 4 query heads do not split in 3
    assert wsz(_prob(Hidx=4), 2) == 0        # 2 index heads per group (w groups 16-byte aligned)
    assert wsz(_prob(Hq=8, Hkv=2, Hidx=16), 4) == 0  # 2 key/value heads neither split in 4 nor shared
    assert wsz(_prob(Hq=8, Hkv=1, Hidx=16), 4) > 0   # one shared key/value head
    ok, f32 = _t(), _t(dtype=sa.SA_F32)
    need = wsz(p, 2)

    def call(g=2, idx=None, ws=FAKE, n=need, pp=p):
        return L.sa_select_attend_grouped(ctypes.byref(pp), g, ok, ok, f32, ok, ok, ok, idx, ok, None, ws, n, None)
    assert call(g=3) == sa.SA_ERR_INVALID_ARG
    assert call(idx=FAKE + 4) == sa.SA_ERR_INVALID_ARG
    assert call(n=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ws=None) == sa.SA_ERR_WORKSPACE


@needs_lib
def test_indexer_argument_errors():
    L = sa.lib()
    p = _prob()
    q = _t(s0=64 * 4 * 32, s1=4 * 32, s2=32)
    k = _t(s0=64 * 32, s1=32, s2=0)
    w = sa._Tensor(FAKE, sa.SA_F32, 64 * 4, 4, 0)
    call = lambda q=q, k=k, w=w, out=FAKE: L.sa_indexer_score(ctypes.byref(p), q, k, w, out, None)
    assert call(out=None) == sa.SA_ERR_INVALID_ARG
    assert call(q=_t(dtype=sa.SA_FP8_E4M3, s0=64 * 4 * 32, s1=4 * 32, s2=32)) == sa.SA_ERR_UNSUPPORTED
    assert call(w=sa._Tensor(FAKE, sa.SA_BF16, 64 * 4, 4, 0)) == sa.SA_ERR_UNSUPPORTED
    assert call(k=_t(data=None, s0=64 * 32, s1=32, s2=0)) == sa.SA_ERR_INVALID_ARG
    assert call(q=_t(s0=64 * 4 * 32, s1=4 * 32, s2=33)) == sa.SA_ERR_INVALID_ARG


@needs_lib
def test_hierarchical_selection_argument_errors():
    L = sa.lib()
    p = _prob()
    q = _t(s0=64 * 4 * 32, s1=4 * 32, s2=32)
    k = _t(s0=64 * 32, s1=32, s2=0)
    w = sa._Tensor(FAKE, sa.SA_F32, 64 * 4, 4, 0)
    ws_need = L.sa_hisa_workspace_bytes(ctypes.byref(p), 16, 2)
    assert ws_need > 0
    assert L.sa_hisa_workspace_bytes(ctypes.byref(p), 24, 2) == 0      # block size not supported
    assert L.sa_hisa_workspace_bytes(ctypes.byref(p), 16, 0) == 0      # no block kept
    assert L.sa_hisa_workspace_bytes(ctypes.byref(p), 128, 2) == 0     # no complete block in the history
    call = lambda blk=16, kb=2, q=q, w=w, kbar=FAKE, idx=FAKE, blocks=None, ws=FAKE, n=ws_need: L.sa_hisa_select(
        ctypes.byref(p), q, k, w, kbar, blk, kb, idx, blocks, ws, n, None)
    assert call(blk=48) == sa.SA_ERR_INVALID_ARG
    assert call(kbar=None) == sa.SA_ERR_INVALID_ARG
    assert call(idx=FAKE + 2) == sa.SA_ERR_INVALID_ARG
    assert call(blocks=FAKE + 2) == sa.SA_ERR_INVALID_ARG
    assert call(n=ws_need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == sa.SA_ERR_WORKSPACE
    # rows of different batches not equally spaced: a row cannot stand as its own batch
    assert call(q=_t(s0=64 * 4 * 32 + 32, s1=4 * 32, s2=32)) == sa.SA_ERR_UNSUPPORTED
    assert call(w=sa._Tensor(FAKE, sa.SA_BF16, 64 * 4, 4, 0)) == sa.SA_ERR_UNSUPPORTED
    bm = lambda blk=16, kb_=k, out=FAKE: L.sa_block_means(ctypes.byref(p), kb_, blk, out, None)
    assert bm(blk=12) == sa.SA_ERR_INVALID_ARG
    assert bm(out=None) == sa.SA_ERR_INVALID_ARG
    assert bm(kb_=_t(data=None, s0=64 * 32, s1=32, s2=0)) == sa.SA_ERR_INVALID_ARG


@needs_lib
@pytest.mark.parametrize("residual", [False, True])
def test_active_head_selection_argument_errors(residual):
    L = sa.lib()
    p = _prob(n_kv=256, Hidx=64, d_idx=64)
    q = _t(s0=64 * 64 * 64, s1=64 * 64, s2=64)
    k = _t(s0=256 * 64, s1=64, s2=0)
    w = sa._Tensor(FAKE, sa.SA_F32, 64 * 64, 64, 0)
    ws_fn = L.sa_resmisa_workspace_bytes if residual else L.sa_misa_workspace_bytes
    fn = L.sa_resmisa_select if residual else L.sa_misa_select
    g_max = 58 if residual else 64  # the shared query takes six of at most 64 scored slots
    assert ws_fn(ctypes.byref(p), 64, g_max) > 0
    assert ws_fn(ctypes.byref(p), 64, g_max + 1) == 0
    assert ws_fn(ctypes.byref(p), 64, 0) == 0
    assert ws_fn(ctypes.byref(p), 512, 4) == 0                          # no complete block
    assert ws_fn(ctypes.byref(_prob(n_kv=256, Hidx=8, d_idx=64)), 64, 4) == 0  # routing: 16, 32 or 64 heads
    need = ws_fn(ctypes.byref(p), 64, 8)
    call = lambda blk=64, g=8, q=q, w=w, kbar=FAKE, idx=FAKE, heads=None, ws=FAKE, n=need: fn(
        ctypes.byref(p), q, k, w, kbar, blk, g, idx, heads, ws, n, None)
    assert call(blk=48) == sa.SA_ERR_INVALID_ARG
    assert call(g=0) == sa.SA_ERR_INVALID_ARG
    assert call(g=g_max + 1) == sa.SA_ERR_INVALID_ARG
    assert call(kbar=FAKE + 8) == sa.SA_ERR_INVALID_ARG
    assert call(idx=None) == sa.SA_ERR_INVALID_ARG
    assert call(heads=FAKE + 2) == sa.SA_ERR_INVALID_ARG
    assert call(q=_t(dtype=sa.SA_F32, s0=64 * 64 * 64, s1=64 * 64, s2=64)) == sa.SA_ERR_UNSUPPORTED
    assert call(n=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == sa.SA_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(sa, "_lib", None)
    monkeypatch.setattr(sa, "LIB_PATH", "/nonexistent/libsa.so")
    with pytest.raises(RuntimeError, match="not built"):
        sa.lib()


@needs_lib
def test_environment_splits_change_the_latent_workspace(monkeypatch):
    # SA_SPLITS sets the latent attention's split count, and with it the partials' space
    L = sa.lib()
    p = sa._Problem(8, 1, 65536, 128, 1, 576, 512, 64, 128, 2048, 1, None, None, 0.0)
    base = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SPARSE_ATTN)
    monkeypatch.setenv("SA_SPLITS", "1")
    one = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SPARSE_ATTN)
    monkeypatch.setenv("SA_SPLITS", "64")  # clamped to one 32-row tile per split
    many = L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SPARSE_ATTN)
    monkeypatch.setenv("SA_SPLITS", "x")  # not a number: ignored
    assert L.sa_workspace_bytes(ctypes.byref(p), sa.SA_OP_SPARSE_ATTN) == base
    assert one < base < many
