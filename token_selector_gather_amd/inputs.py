"""Move a host workload (numpy arrays from the seeded generator) into device tensors.

Storage dtypes map as float32 -> torch.float32, uint16 (bf16 bit patterns) ->
torch.bfloat16 and uint8 (OCP e4m3fn codes) -> torch.float8_e4m3fn; the bytes are
copied unchanged.
"""
import numpy as np
import torch

from . import Problem

_VIEW = {np.dtype(np.float32): torch.float32, np.dtype(np.uint16): torch.bfloat16,
         np.dtype(np.uint8): torch.float8_e4m3fn}


def to_device(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    elif a.dtype == np.uint8:
        t = torch.from_numpy(a).to(device).view(torch.float8_e4m3fn)
    elif a.dtype == np.float32:
        t = torch.from_numpy(a).to(device)
    elif a.dtype == np.int32:
        t = torch.from_numpy(a).to(device)
    else:
        raise TypeError(a.dtype)
    return t


def device_workload(W, device="cuda", with_main=True):
    """Returns (Problem, dict of device tensors) for a workload dict from sa_synth.make_config."""
    d = {}
    d["kv_len"] = to_device(np.asarray(W["kv_len"], np.int32), device)
    d["q_pos0"] = to_device(np.asarray(W["q_pos0"], np.int32), device)
    for key in ("q_idx", "k_idx", "w"):
        d[key] = to_device(W[key], device)
    if with_main:
        d["Q"] = to_device(W["Q"], device)
        d["K"] = to_device(W["K"], device)
        d["V"] = to_device(W["V"], device) if W.get("V") is not None else d["K"][..., : W["d_v"]]
    P = Problem(W["B"], W["n_q"], W["n_kv"], W["Hq"], W["Hkv"], W["d_qk"], W["d_v"], W["Hidx"], W["d_idx"],
                W["k"], W["causal"], kv_len=d["kv_len"], q_pos0=d["q_pos0"], scale=W["scale"])
    return P, d


def empty_outputs(W, dtype, device="cuda"):
    B, Hq, nq, dv, k = W["B"], W["Hq"], W["n_q"], W["d_v"], W["k"]
    O = torch.full((B, Hq, nq, dv), float("nan"), dtype=dtype, device=device)
    lse = torch.full((B, Hq, nq), float("nan"), dtype=torch.float32, device=device)
    idx = torch.full((B, nq, k), -7, dtype=torch.int32, device=device)
    return O, lse, idx


def device_pool(X, block_table, page_size, pool_rows, fill=3.0e4, check_rows=256, seed=0):
    """Paged copy of per-batch device rows X [B, H, n_kv, d]: a pool [1, H, pool_rows, d] in
    which logical row j of batch b is row block_table[b, j // page_size] * page_size +
    j % page_size; rows no batch uses hold `fill`.  Pages are copied as slices (no indexed
    scatter over the whole pool), then `check_rows` random rows and each batch's last row
    are compared with their sources."""
    B, H, n_kv, d = X.shape
    bt = np.asarray(block_table, np.int64)
    npg = -(-n_kv // page_size)
    if bt.min(initial=0) < 0 or (bt[:, :npg].max(initial=0) + 1) * page_size > pool_rows:
        raise ValueError("device_pool: the block table names rows outside the pool")
    pool = torch.full((1, H, pool_rows, d), fill, dtype=X.dtype, device=X.device)
    for b in range(B):
        for pg in range(npg):
            lo, dst = pg * page_size, int(bt[b, pg]) * page_size
            hi = min(lo + page_size, n_kv)
            pool[0, :, dst:dst + hi - lo].copy_(X[b, :, lo:hi])
    rng = np.random.default_rng(seed)
    bs = np.concatenate([rng.integers(0, B, check_rows), np.arange(B)])
    js = np.concatenate([rng.integers(0, n_kv, check_rows), np.full(B, n_kv - 1)])
    for b, j in zip(bs.tolist(), js.tolist()):
        r = int(bt[b, j // page_size]) * page_size + j % page_size
        if not torch.equal(pool[0, :, r], X[b, :, j]):
            raise RuntimeError("device_pool: pool row %d does not hold batch %d position %d" % (r, b, j))
    return pool
