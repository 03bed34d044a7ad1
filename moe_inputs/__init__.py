"""Seeded synthetic inputs shared by the float64 oracle and the GPU path.

Nothing here computes any step of the MoE layer: the module draws numbers and
stores them in the byte formats the layer step consumes (see ``gen.c`` for the
generator and the expert-blob layout).  The C part is compiled on first use
into ``libmoe_inputs.so`` beside this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .workloads import WORKLOADS, Workload, blob_bytes  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_SRC_NORMALS = os.path.join(_HERE, "normals.c")
_LIB = os.path.join(_HERE, "libmoe_inputs.so")
_lock = threading.Lock()
_lib = None

FMT_BF16, FMT_FP8, FMT_MXFP4 = 0, 1, 2
PURPOSE_ROUTER, PURPOSE_EXPERT, PURPOSE_SHARED, PURPOSE_DECODE, PURPOSE_PREFILL = 1, 2, 3, 4, 5


def _stale() -> bool:
    if not os.path.exists(_LIB):
        return True
    t = os.path.getmtime(_LIB)
    return t < os.path.getmtime(_SRC) or t < os.path.getmtime(_SRC_NORMALS)


def build(force: bool = False) -> str:
    """Compile gen.c + normals.c into libmoe_inputs.so (gcc, OpenMP, libmvec).

    normals.c is built with -ffast-math and AVX2 so its log/sin/cos vectorise; the
    encoders in gen.c are built without fast-math."""
    if force or _stale():
        tag = f"{os.getpid()}"
        on = os.path.join(_HERE, f"normals.{tag}.o")
        og = os.path.join(_HERE, f"gen.{tag}.o")
        tmp = _LIB + f".tmp{tag}"
        try:
            subprocess.check_call(["gcc", "-O3", "-ffast-math", "-mavx2", "-mfma", "-fPIC", "-c",
                                   _SRC_NORMALS, "-o", on])
            subprocess.check_call(["gcc", "-O3", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-c", _SRC, "-o", og])
            subprocess.check_call(["gcc", "-shared", "-fopenmp", "-o", tmp, og, on, "-lmvec", "-lm"])
            os.replace(tmp, _LIB)
        finally:
            for f in (on, og, tmp):
                if os.path.exists(f):
                    os.remove(f)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _stale():
                build()
            lib = ctypes.CDLL(_LIB)
            u64, i64, u32, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int
            vp = ctypes.c_void_p
            lib.moe_in_stream_key.restype = u64
            lib.moe_in_stream_key.argtypes = [u64, u32, u32, u32, u32]
            lib.moe_in_draw.restype = u64
            lib.moe_in_draw.argtypes = [u64, u64]
            lib.moe_in_normals.argtypes = [u64, u64, u64, vp]
            lib.moe_in_enc_e4m3.restype = ctypes.c_uint8
            lib.moe_in_enc_e4m3.argtypes = [ctypes.c_float]
            lib.moe_in_enc_e2m1.restype = ctypes.c_uint8
            lib.moe_in_enc_e2m1.argtypes = [ctypes.c_float]
            lib.moe_in_blob_bytes.restype = i64
            lib.moe_in_blob_bytes.argtypes = [i32, i64, i64]
            lib.moe_in_expert_f32.argtypes = [u64, u32, u32, u32, i64, i64, vp, vp, vp]
            lib.moe_in_expert_blob.argtypes = [u64, i32, u32, u32, u32, i64, i64, vp]
            lib.moe_in_pool.argtypes = [u64, i32, i64, i64, i64, i64, i64, vp, i32]
            lib.moe_in_router.argtypes = [u64, i64, i64, i64, i64, vp, i32]
            lib.moe_in_decode_acts.argtypes = [u64, i64, i64, i64, i64, i64, vp, i32]
            lib.moe_in_prefill_acts.argtypes = [u64, i64, i64, i64, i64, vp, i32]
            _lib = lib
    return _lib


def _ptr(a) -> int:
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    return int(a)


def stream_key(seed, purpose, layer, unit, matrix) -> int:
    return _load().moe_in_stream_key(seed, purpose, layer, unit, matrix)


def normals(key: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().moe_in_normals(key, first, n, _ptr(out))
    return out


def enc_e4m3(x: float) -> int:
    return int(_load().moe_in_enc_e4m3(x))


def enc_e2m1(x: float) -> int:
    return int(_load().moe_in_enc_e2m1(x))


def expert_f32(seed, purpose, layer, unit, H, I):
    """fp32 weights before encoding (Wg [I,H], Wu [I,H], Wd [H,I]) of one expert."""
    Wg = np.empty((I, H), np.float32); Wu = np.empty((I, H), np.float32)
    Wd = np.empty((H, I), np.float32)
    _load().moe_in_expert_f32(seed, purpose, layer, unit, H, I, _ptr(Wg), _ptr(Wu), _ptr(Wd))
    return Wg, Wu, Wd


def expert_blob(seed, fmt, purpose, layer, unit, H, I, out=None) -> np.ndarray:
    S = blob_bytes(fmt, H, I)
    if out is None:
        out = np.empty(S, dtype=np.uint8)
    _load().moe_in_expert_blob(seed, fmt, purpose, layer, unit, H, I, _ptr(out))
    return out


def fill_pool(seed, fmt, l0, nl, E, H, I, dst, nthreads: int = 0) -> None:
    """Write the blobs of layers [l0, l0+nl) x E experts to ``dst`` (numpy array or raw address)."""
    _load().moe_in_pool(seed, fmt, l0, nl, E, H, I, _ptr(dst), nthreads)


def router_weights(seed, l0, nl, E, H, out=None, nthreads: int = 0) -> np.ndarray:
    if out is None:
        out = np.empty((nl, E, H), dtype=np.uint16)
    _load().moe_in_router(seed, l0, nl, E, H, _ptr(out), nthreads)
    return out


def decode_acts(seed, l0, nl, S, ntok, H, out=None, nthreads: int = 0) -> np.ndarray:
    """bf16 AR(1) activations, shape [ntok, nl, S, H] (token, layer, stream, hidden)."""
    if out is None:
        out = np.empty((ntok, nl, S, H), dtype=np.uint16)
    _load().moe_in_decode_acts(seed, l0, nl, S, ntok, H, _ptr(out), nthreads)
    return out


def prefill_acts(seed, l0, nl, T, H, out=None, nthreads: int = 0) -> np.ndarray:
    """bf16 i.i.d. N(0,1) activations, shape [nl, T, H]."""
    if out is None:
        out = np.empty((nl, T, H), dtype=np.uint16)
    _load().moe_in_prefill_acts(seed, l0, nl, T, H, _ptr(out), nthreads)
    return out


def shared_blob(seed, fmt, layer, H, I, out=None) -> np.ndarray:
    return expert_blob(seed, fmt, PURPOSE_SHARED, layer, 0, H, I, out)
