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
