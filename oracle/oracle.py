"""ctypes driver for the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark; never by the library.

Storage dtypes are inferred from numpy arrays: float32 -> f32, uint16 -> bf16 bit
patterns, uint8 -> OCP FP8 e4m3fn codes.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, E4M3 = 0, 1, 2


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "n_q", "n_kv", "Hq", "Hkv", "d_qk", "d_v", "Hidx", "d_idx", "k", "causal")] + [
        ("scale", ctypes.c_double),
        ("kv_len", ctypes.c_void_p),
        ("q_pos0", ctypes.c_void_p),
        ("pos_of_slot", ctypes.c_void_p),
    ]


class _View(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("s0", ctypes.c_int64), ("s1", ctypes.c_int64), ("s2", ctypes.c_int64)]


def build(force=False):
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, src, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P, V = ctypes.POINTER(_Problem), _View
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.or_scores.argtypes = [P, V, V, V, i64, vp, vp, i32]
        L.or_scores.restype = i32
        L.or_select.argtypes = [P, vp, i64, vp, vp, vp, vp, vp, i32]
        L.or_select.restype = None
        L.or_attend.argtypes = [P, V, V, V, vp, i64, i64, vp, vp, vp, i32]
        L.or_attend.restype = i32
        L.or_count_visible.argtypes = [P]
        L.or_count_visible.restype = ctypes.c_int64
        L.or_decode_one.argtypes = [i32, ctypes.c_uint32]
        L.or_decode_one.restype = ctypes.c_double
        _lib = L
    return _lib


def threads():
    return max(1, min(64, os.cpu_count() or 1))


def _dtype_code(a):
    return {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): E4M3}[a.dtype]


def _view(a, ncols=None):
    """Strided view of a numpy array whose last dimension is contiguous; 2-, 3- and
    4-d arrays map to (s0, s1, s2) element strides of their leading dimensions."""
    assert a.strides[-1] == a.itemsize, "last dimension must be contiguous"
    st = [s // a.itemsize for s in a.strides[:-1]]
    st = st + [0] * (3 - len(st))
    return _View(a.ctypes.data, _dtype_code(a), st[0], st[1], st[2])


class Problem:
    """Keeps the ctypes problem struct and the host arrays it points into alive."""

    def __init__(self, W, pos_of_slot=None, k=None, causal=None, scale=None):
        self.kv_len = np.ascontiguousarray(W["kv_len"], dtype=np.int32)
        self.q_pos0 = np.ascontiguousarray(W["q_pos0"], dtype=np.int32)
        self.pos = None if pos_of_slot is None else np.ascontiguousarray(pos_of_slot, dtype=np.int32)
        s = W["scale"] if scale is None else scale
        self.p = _Problem(W["B"], W["n_q"], W["n_kv"], W["Hq"], W["Hkv"], W["d_qk"], W["d_v"], W["Hidx"],
                          W["d_idx"], W["k"] if k is None else k, W["causal"] if causal is None else causal,
                          float(s), self.kv_len.ctypes.data, self.q_pos0.ctypes.data,
                          None if self.pos is None else self.pos.ctypes.data)
        self.k = self.p.k


def _rows(W, rows):
    if rows is None:
        rows = np.arange(W["B"] * W["n_q"], dtype=np.int32)
    return np.ascontiguousarray(rows, dtype=np.int32)


def scores(W, rows=None, pos_of_slot=None, k_idx=None):
    """fp64 indexer scores [len(rows), n_kv]; -inf where not visible."""
    P = Problem(W, pos_of_slot)
    rows = _rows(W, rows)
    q, kk, w = W["q_idx"], W["k_idx"] if k_idx is None else k_idx, W["w"]
    out = np.empty((rows.size, W["n_kv"]), dtype=np.float64)
    rc = lib().or_scores(ctypes.byref(P.p), _view(q), _view(kk), _view(w), rows.size, rows.ctypes.data,
                         out.ctypes.data, threads())
    if rc != 0:
        raise ValueError("oracle: non-finite index input")
    return out


def select(W, sc, rows=None, pos_of_slot=None, k=None):
    """Top-k of given fp64 score rows.  Returns (idx int32 [n,k], s_k, s_k+1, n_selected)."""
    P = Problem(W, pos_of_slot, k=k)
    rows = _rows(W, rows)
    sc = np.ascontiguousarray(sc, dtype=np.float64)
    assert sc.shape == (rows.size, W["n_kv"])
    n = rows.size
    idx = np.empty((n, P.k), dtype=np.int32)
    sk, skp1 = np.empty(n), np.empty(n)
    nsel = np.empty(n, dtype=np.int32)
    lib().or_select(ctypes.byref(P.p), sc.ctypes.data, n, rows.ctypes.data, idx.ctypes.data, sk.ctypes.data,
                    skp1.ctypes.data, nsel.ctypes.data, threads())
    return idx, sk, skp1, nsel


def attend(W, idx, rows=None, pos_of_slot=None, Q=None, K=None, V=None, scale=None):
    """fp64 softmax attention of the listed rows over idx ([n, k] slots, -1 skipped).
    Returns (O [n, Hq, d_v], lse [n, Hq])."""
    P = Problem(W, pos_of_slot, k=np.asarray(idx).shape[1], scale=scale)
    rows = _rows(W, rows)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Q = W["Q"] if Q is None else Q
    K = W["K"] if K is None else K
    V = W["V"] if V is None else V
    if V is None:  # latent layout: V is the first d_v columns of each K row
        V = K[..., : W["d_v"]]
    n = rows.size
    O = np.empty((n, W["Hq"], W["d_v"]), dtype=np.float64)
    lse = np.empty((n, W["Hq"]), dtype=np.float64)
    rc = lib().or_attend(ctypes.byref(P.p), _view(Q), _view(K), _view(V), idx.ctypes.data, idx.shape[1], n,
                         rows.ctypes.data, O.ctypes.data, lse.ctypes.data, threads())
    if rc != 0:
        raise ValueError("oracle: non-finite attention input")
    return O, lse


def count_visible(W, causal=None):
    P = Problem(W, causal=causal)
    return lib().or_count_visible(ctypes.byref(P.p))


def decode(dtype, bits):
    return lib().or_decode_one(dtype, int(bits))


def select_attend(W, rows=None):
    """Full path on the listed rows: scores -> select -> attention."""
    rows = _rows(W, rows)
    sc = scores(W, rows)
    idx, sk, skp1, nsel = select(W, sc, rows)
    O, lse = attend(W, idx, rows)
    return dict(scores=sc, idx=idx, sk=sk, skp1=skp1, nsel=nsel, O=O, lse=lse)
