"""Seeded synthetic inputs shared by the GPU library's tests/bench and the CPU oracle.

The random stream, Box-Muller normals and the bf16 / OCP-e4m3fn encoders live in
``synth.c`` (built with gcc into ``libsasynth.so``).  This module only marshals
arguments and assembles the five workload configurations.  It contains none of
the method's arithmetic (no indexer score, no selection, no softmax).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsasynth.so")
_lib = None

F32, BF16, E4M3, F64 = 0, 1, 2, 3
NP_STORAGE = {F32: np.float32, BF16: np.uint16, E4M3: np.uint8, F64: np.float64}
DTYPE_NAMES = {F32: "f32", BF16: "bf16", E4M3: "e4m3"}


def build(force=False):
    """Compile synth.c with gcc (CPU only)."""
    src = os.path.join(_HERE, "synth.c")
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
        u64, i64, dbl, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        L.syn_normal.argtypes = [u64, u64, i64, i64, dbl, dbl, i32, vp, i32]
        L.syn_uniform.argtypes = [u64, u64, i64, i64, dbl, dbl, i32, vp, i32]
        L.syn_encode.argtypes = [vp, i64, i32, vp, i32]
        for f in (L.syn_normal, L.syn_uniform, L.syn_encode):
            f.restype = None
        _lib = L
    return _lib


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def normal(seed, tid, shape, dtype, scale=1.0, shift=0.0, off=0):
    out = np.empty(shape, dtype=NP_STORAGE[dtype])
    lib().syn_normal(seed, tid, off, out.size, scale, shift, dtype, out.ctypes.data, _threads())
    return out


def uniform(seed, tid, shape, dtype, lo=0.0, hi=1.0, off=0):
    out = np.empty(shape, dtype=NP_STORAGE[dtype])
    lib().syn_uniform(seed, tid, off, out.size, lo, hi, dtype, out.ctypes.data, _threads())
    return out


def encode(values, dtype):
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=NP_STORAGE[dtype])
    lib().syn_encode(v.ctypes.data, v.size, dtype, out.ctypes.data, _threads())
    return out


def bf16_to_f32(a):
    """Widen stored bf16 bit patterns (uint16) to float32 (exact)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


from .configs import CONFIGS, custom, make_config, paged_layout, poison_value, to_pool  # noqa: E402,F401
