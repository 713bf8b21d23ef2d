"""Python binding of libsa.so: content-routed token-sparse attention on MI355X (gfx950).

Argument marshalling only.  Every step of the path (indexer score, top-k selection,
sparse gather attention) runs in the HIP kernels of libsa.so; PyTorch supplies device
memory and the stream.  Importing works without a GPU; every call needs the built
library and raises if it is missing.

The functions mirror the C ABI in include/sa.h and keep its names:
    sa_indexer_score, sa_topk, sa_select, sa_sparse_attn, sa_select_attend,
    sa_block_means, sa_hisa_select, sa_hisa_workspace_bytes, sa_misa_select, sa_misa_workspace_bytes,
    sa_workspace_bytes, sa_device_status, sa_status_str, sa_abi_version
Tensors are torch tensors on the GPU whose last dimension is contiguous: float32,
bfloat16 or float8_e4m3fn (index keys only).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsa.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP, SA_ERR_NONFINITE, SA_ERR_INDEX = range(7)
SA_F32, SA_BF16, SA_FP8_E4M3 = 0, 1, 2
SA_OP_INDEXER_SCORE, SA_OP_TOPK, SA_OP_SPARSE_ATTN, SA_OP_SELECT_ATTEND, SA_OP_SPARSE_ATTN_PAGED, SA_OP_SELECT = range(6)
ABI_VERSION = 2

_TORCH_DTYPES = {torch.float32: SA_F32, torch.bfloat16: SA_BF16, torch.float8_e4m3fn: SA_FP8_E4M3}


class SaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s" % (what, sa_status_str(status)))


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("s0", ctypes.c_int64), ("s1", ctypes.c_int64), ("s2", ctypes.c_int64)]


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "n_q", "n_kv", "Hq", "Hkv", "d_qk", "d_v", "Hidx", "d_idx", "k", "causal")] + [
        ("kv_len", ctypes.c_void_p), ("q_pos0", ctypes.c_void_p), ("scale", ctypes.c_float)]


_lib = None


def lib():
    """The loaded libsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsa.so is not built (build it with token_selector_gather_amd.build.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        T, P, vp, sz, i64 = _Tensor, ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
        st = ctypes.c_int
        L.sa_indexer_score.argtypes = [P, T, T, T, vp, vp]
        L.sa_topk.argtypes = [P, vp, i64, vp, vp, vp, sz, vp]
        L.sa_select.argtypes = [P, T, T, T, vp, vp, sz, vp]
        L.sa_sparse_attn.argtypes = [P, T, T, T, vp, T, vp, vp, sz, vp]
        L.sa_select_attend.argtypes = [P, T, T, T, T, T, T, vp, T, vp, vp, sz, vp]
        L.sa_select_attend_noalloc.argtypes = [P, T, T, T, T, T, T, vp, T, vp, vp, vp]
        L.sa_sparse_attn_paged.argtypes = [P, T, T, T, i64, vp, i64, ctypes.c_int, vp, T, vp, vp, sz, vp]
        L.sa_select_attend_grouped.argtypes = [P, ctypes.c_int, T, T, T, T, T, T, vp, T, vp, vp, sz, vp]
        L.sa_grouped_workspace_bytes.argtypes = [P, ctypes.c_int]
        L.sa_grouped_workspace_bytes.restype = sz
        L.sa_block_means.argtypes = [P, T, ctypes.c_int, vp, vp]
        L.sa_hisa_select.argtypes = [P, T, T, T, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, sz, vp]
        L.sa_misa_select.argtypes = [P, T, T, T, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, sz, vp]
        L.sa_resmisa_select.argtypes = [P, T, T, T, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, sz, vp]
        for f in (L.sa_indexer_score, L.sa_topk, L.sa_select, L.sa_sparse_attn, L.sa_select_attend,
                  L.sa_select_attend_noalloc, L.sa_block_means,
                  L.sa_hisa_select, L.sa_misa_select, L.sa_resmisa_select, L.sa_sparse_attn_paged, L.sa_select_attend_grouped):
            f.restype = st
        L.sa_misa_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int]
        L.sa_misa_workspace_bytes.restype = sz
        L.sa_resmisa_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int]
        L.sa_resmisa_workspace_bytes.restype = sz
        L.sa_hisa_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int]
        L.sa_hisa_workspace_bytes.restype = sz
        L.sa_workspace_bytes.argtypes = [P, ctypes.c_int]
        L.sa_workspace_bytes.restype = sz
        L.sa_device_status.argtypes = [vp, vp]
        L.sa_device_status.restype = st
        L.sa_status_str.argtypes = [st]
        L.sa_status_str.restype = ctypes.c_char_p
        L.sa_abi_version.argtypes = []
        L.sa_abi_version.restype = ctypes.c_int
        if L.sa_abi_version() != ABI_VERSION:
            raise RuntimeError("libsa.so ABI version %d, binding expects %d" % (L.sa_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


class Problem:
    """Problem sizes plus the device int32 tensors kv_len [B] and q_pos0 [B] (either may be None)."""

    FIELDS = ("B", "n_q", "n_kv", "Hq", "Hkv", "d_qk", "d_v", "Hidx", "d_idx", "k", "causal")

    def __init__(self, B, n_q, n_kv, Hq, Hkv, d_qk, d_v, Hidx, d_idx, k, causal=1, kv_len=None, q_pos0=None,
                 scale=0.0):
        self.kv_len, self.q_pos0 = kv_len, q_pos0
        for t in (kv_len, q_pos0):
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise ValueError("kv_len / q_pos0 must be contiguous int32 tensors")
        self.c = _Problem(B, n_q, n_kv, Hq, Hkv, d_qk, d_v, Hidx, d_idx, k, int(causal),
                          kv_len.data_ptr() if kv_len is not None else None,
                          q_pos0.data_ptr() if q_pos0 is not None else None, float(scale))
        for f in self.FIELDS:
            setattr(self, f, getattr(self.c, f))
        self.scale = scale

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _tensor(t, what):
    if t is None:
        return _Tensor(None, 0, 0, 0, 0)
    if t.dtype not in _TORCH_DTYPES:
        raise TypeError("%s: unsupported dtype %s" % (what, t.dtype))
    if t.stride(-1) != 1:
        raise ValueError("%s: last dimension must be contiguous" % what)
    st = list(t.stride()[:-1]) + [0, 0, 0]
    return _Tensor(t.data_ptr(), _TORCH_DTYPES[t.dtype], st[0], st[1], st[2])


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, what):
    if status != SA_OK:
        raise SaError(status, what)


def sa_status_str(status):
    return lib().sa_status_str(status).decode()


def sa_abi_version():
    return lib().sa_abi_version()


def sa_workspace_bytes(p, op):
    return lib().sa_workspace_bytes(p.ref, op)


def workspace(p, op, device="cuda"):
    """A zero-filled workspace of the size sa_workspace_bytes(p, op) asks for."""
    n = max(256, sa_workspace_bytes(p, op))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sa_indexer_score(p, q_idx, k_idx, w, scores, stream=None):
    _check(lib().sa_indexer_score(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"),
                                  _ptr(scores), _stream(stream)), "sa_indexer_score")


def sa_topk(p, scores, row_stride, idx, vals, ws, stream=None):
    _check(lib().sa_topk(p.ref, _ptr(scores), int(row_stride), _ptr(idx), _ptr(vals), _ptr(ws),
                         0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "sa_topk")


def sa_select(p, q_idx, k_idx, w, idx, ws, stream=None):
    _check(lib().sa_select(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"), _ptr(idx),
                           _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_select")


def sa_sparse_attn(p, Q, K, V, idx, O, lse, ws, stream=None):
    _check(lib().sa_sparse_attn(p.ref, _tensor(Q, "Q"), _tensor(K, "K"), _tensor(V, "V"), _ptr(idx),
                                _tensor(O, "O"), _ptr(lse), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_sparse_attn")


def sa_sparse_attn_paged(p, Q, K_pool, V_pool, block_table, page_size, idx, O, lse, ws, stream=None):
    """sa_sparse_attn over paged pools K_pool / V_pool [1, Hkv, pool_rows, d] (one unit leading
    dimension, so that the head and row strides land where the C call reads them) and an int32
    block_table [B, pages per batch]."""
    if K_pool.dim() != 4 or K_pool.shape[0] != 1 or V_pool.dim() != 4 or V_pool.shape[0] != 1:
        raise ValueError("K_pool and V_pool must be [1, Hkv, pool_rows, d]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be an int32 [B, pages] tensor with contiguous rows")
    _check(lib().sa_sparse_attn_paged(p.ref, _tensor(Q, "Q"), _tensor(K_pool, "K_pool"), _tensor(V_pool, "V_pool"),
                                      int(K_pool.shape[2]), _ptr(block_table), int(block_table.stride(0)),
                                      int(page_size), _ptr(idx), _tensor(O, "O"), _ptr(lse), _ptr(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_sparse_attn_paged")


def sa_select_attend(p, q_idx, k_idx, w, Q, K, V, idx_out, O, lse, ws, stream=None):
    _check(lib().sa_select_attend(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"),
                                  _tensor(Q, "Q"), _tensor(K, "K"), _tensor(V, "V"), _ptr(idx_out),
                                  _tensor(O, "O"), _ptr(lse), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_select_attend")


def sa_select_attend_noalloc(p, q_idx, k_idx, w, Q, K, V, idx_out, O, lse, status=None, stream=None):
    """sa_select_attend on the library's fixed device scratch (no workspace argument); status
    is a zero-filled 256-byte device tensor or None."""
    _check(lib().sa_select_attend_noalloc(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"),
                                          _tensor(Q, "Q"), _tensor(K, "K"), _tensor(V, "V"), _ptr(idx_out),
                                          _tensor(O, "O"), _ptr(lse), _ptr(status), _stream(stream)),
           "sa_select_attend_noalloc")


def sa_grouped_workspace_bytes(p, groups):
    return lib().sa_grouped_workspace_bytes(p.ref, int(groups))


def grouped_workspace(p, groups, device="cuda"):
    """A zero-filled workspace for sa_select_attend_grouped."""
    n = max(256, sa_grouped_workspace_bytes(p, groups))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sa_select_attend_grouped(p, groups, q_idx, k_idx, w, Q, K, V, idx_out, O, lse, ws, stream=None):
    """Grouped candidate sets; idx_out is [groups, B, n_q, k] int32 or None."""
    _check(lib().sa_select_attend_grouped(p.ref, int(groups), _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"),
                                          _tensor(w, "w"), _tensor(Q, "Q"), _tensor(K, "K"), _tensor(V, "V"),
                                          _ptr(idx_out), _tensor(O, "O"), _ptr(lse), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_select_attend_grouped")


def sa_block_means(p, k_idx, blk, kbar, stream=None):
    """Block representatives kbar [B, n_kv // blk, d_idx] (bf16 tensor) of k_idx."""
    if kbar.dtype != torch.bfloat16 or not kbar.is_contiguous():
        raise ValueError("kbar must be a contiguous bfloat16 tensor")
    _check(lib().sa_block_means(p.ref, _tensor(k_idx, "k_idx"), int(blk), _ptr(kbar), _stream(stream)),
           "sa_block_means")


def sa_hisa_workspace_bytes(p, blk, k_blocks):
    return lib().sa_hisa_workspace_bytes(p.ref, int(blk), int(k_blocks))


def hisa_workspace(p, blk, k_blocks, device="cuda"):
    """A zero-filled workspace for sa_hisa_select."""
    n = max(256, sa_hisa_workspace_bytes(p, blk, k_blocks))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sa_hisa_select(p, q_idx, k_idx, w, kbar, blk, k_blocks, idx, ws, blocks=None, stream=None):
    _check(lib().sa_hisa_select(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"), _ptr(kbar),
                                int(blk), int(k_blocks), _ptr(idx), _ptr(blocks), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_hisa_select")


def sa_misa_workspace_bytes(p, blk, g):
    return lib().sa_misa_workspace_bytes(p.ref, int(blk), int(g))


def misa_workspace(p, blk, g, device="cuda"):
    """A zero-filled workspace for sa_misa_select."""
    n = max(256, sa_misa_workspace_bytes(p, blk, g))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sa_misa_select(p, q_idx, k_idx, w, kbar, blk, g, idx, ws, heads=None, stream=None):
    _check(lib().sa_misa_select(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"), _ptr(kbar),
                                int(blk), int(g), _ptr(idx), _ptr(heads), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_misa_select")


def sa_resmisa_workspace_bytes(p, blk, g):
    return lib().sa_resmisa_workspace_bytes(p.ref, int(blk), int(g))


def resmisa_workspace(p, blk, g, device="cuda"):
    """A zero-filled workspace for sa_resmisa_select."""
    n = max(256, sa_resmisa_workspace_bytes(p, blk, g))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sa_resmisa_select(p, q_idx, k_idx, w, kbar, blk, g, idx, ws, heads=None, stream=None):
    _check(lib().sa_resmisa_select(p.ref, _tensor(q_idx, "q_idx"), _tensor(k_idx, "k_idx"), _tensor(w, "w"),
                                   _ptr(kbar), int(blk), int(g), _ptr(idx), _ptr(heads), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "sa_resmisa_select")


def sa_device_status(ws, stream=None):
    """Synchronises, returns and clears the device status word kept in ws."""
    return lib().sa_device_status(_ptr(ws), _stream(stream))
