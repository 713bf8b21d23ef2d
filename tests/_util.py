"""Helpers shared by the tests: hand-built tiny workloads in f32 storage."""
import math

import numpy as np


def tiny(Q=None, K=None, V=None, q_idx=None, k_idx=None, w=None, k=4, causal=1, scale=1.0,
         kv_len=None, q_pos0=None):
    """Workload dict from explicit float arrays (stored as f32).
    Q [B,Hq,n_q,d], K [B,Hkv,n_kv,d], V [B,Hkv,n_kv,dv], q_idx [B,n_q,H,di], k_idx [B,n_kv,di], w [B,n_q,H]."""
    f = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    Q, K, V, q_idx, k_idx, w = map(f, (Q, K, V, q_idx, k_idx, w))
    src = Q if Q is not None else q_idx
    B = src.shape[0]
    n_q = Q.shape[2] if Q is not None else q_idx.shape[1]
    n_kv = K.shape[2] if K is not None else k_idx.shape[1]
    W = dict(B=B, n_q=n_q, n_kv=n_kv, k=k, causal=causal, scale=scale,
             Hq=Q.shape[1] if Q is not None else 1, Hkv=K.shape[1] if K is not None else 1,
             d_qk=Q.shape[3] if Q is not None else 1, d_v=V.shape[3] if V is not None else 1,
             Hidx=q_idx.shape[2] if q_idx is not None else 1, d_idx=q_idx.shape[3] if q_idx is not None else 1,
             Q=Q, K=K, V=V, q_idx=q_idx, k_idx=k_idx, w=w)
    W["kv_len"] = np.full(B, n_kv, np.int32) if kv_len is None else np.asarray(kv_len, np.int32)
    W["q_pos0"] = np.zeros(B, np.int32) if q_pos0 is None else np.asarray(q_pos0, np.int32)
    return W


def all_rows(W):
    return np.arange(W["B"] * W["n_q"], dtype=np.int32)


def full_idx(W, rows=None):
    """Index lists naming every history slot 0..n_kv-1 (the mask decides visibility)."""
    n = W["B"] * W["n_q"] if rows is None else len(rows)
    return np.tile(np.arange(W["n_kv"], dtype=np.int32), (n, 1))


def rand_f32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def approx_eq(a, b, tol):
    return abs(a - b) <= tol


LN = math.log
