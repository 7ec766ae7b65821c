"""CPU oracle for the routed-expert MoE decode path (fp64, plain C).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may use this package; the product path never
does.  It shares no code with the HIP library; the two read the same input
bytes produced by ``synth``.

Functions whose result is pinned by tests other than the GPU comparison are
listed in the tests (closed forms, brute force, invariants, hand-simulated
traces).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-Wextra", "-Wno-unused-parameter", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = D
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = D
        L.oracle_record_layout.argtypes = [I32, I32, P, P, P, P]
        L.oracle_code_pair.argtypes = [P, I32, I32, I32]
        L.oracle_code_pair.restype = ctypes.c_uint32
        L.oracle_rvq_decode_row.argtypes = [P, P, P, I32, I32, I32, P]
        L.oracle_rvq_gemv.argtypes = [P, P, P, I32, I32, P, I32, P]
        L.oracle_expert_ffn.argtypes = [P, I32, I32, P, I32, P]
        L.oracle_shared_ffn.argtypes = [P, I32, I32, P, I32, P]
        L.oracle_route.argtypes = [P, P, I32, I32, P, I32, I32, I32, P, P, P]
        L.oracle_layer.argtypes = [P, P, I32, I32, I32, P, P, I32, I32, P, I32, P, P, P]
        L.oracle_lru.argtypes = [P, I64, I32, P, P, P]
        L.oracle_stream_trace.argtypes = [P, I64, I32, I32, I32, I32, I32, P, P, P, P]
        L.oracle_two_tier.argtypes = [P, I64, I32, I32, P, P, P, P, P, P, P]
        L.oracle_set_threads.argtypes = [I32]
        L.oracle_get_threads.restype = I32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


SCORE = {"softmax": 0, "sigmoid": 1}


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return lib().oracle_get_threads()


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def record_layout(H: int, I: int):
    off = np.zeros(9, np.int64)
    size = np.zeros(9, np.int64)
    nb = np.zeros(1, np.int64)
    pad = np.zeros(1, np.int64)
    _check(lib().oracle_record_layout(H, I, _p(off), _p(size), _p(nb), _p(pad)), "layout")
    return off, size, int(nb[0]), int(pad[0])


def code_pair(section: np.ndarray, K: int, r: int, q: int) -> int:
    s = _c(section, np.uint8)
    return int(lib().oracle_code_pair(_p(s), K, r, q))


def decode_row(section, scales, codebook, N: int, K: int, r: int) -> np.ndarray:
    s, sc, cb = _c(section, np.uint8), _c(scales, np.float16), _c(codebook, np.float16)
    w = np.zeros(K, np.float64)
    _check(lib().oracle_rvq_decode_row(_p(s), _p(sc), _p(cb), N, K, r, _p(w)), "decode_row")
    return w


def rvq_gemv(section, scales, codebook, N: int, K: int, x) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float64)
    s, sc, cb = _c(section, np.uint8), _c(scales, np.float16), _c(codebook, np.float16)
    y = np.zeros((x.shape[0], N), np.float64)
    _check(lib().oracle_rvq_gemv(_p(s), _p(sc), _p(cb), N, K, _p(x), x.shape[0], _p(y)), "gemv")
    return y


def expert_ffn(record, H: int, I: int, x) -> np.ndarray:
    """y [T, H] = W_d (SiLU(W_g x) * W_u x) for one RVQ expert record."""
    x = _c(np.atleast_2d(x), np.float64)
    rec = _c(record, np.uint8)
    y = np.zeros((x.shape[0], H), np.float64)
    _check(lib().oracle_expert_ffn(_p(rec), H, I, _p(x), x.shape[0], _p(y)), "expert_ffn")
    return y


def shared_ffn(shared_bits, H: int, I: int, x) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float64)
    w = _c(shared_bits, np.uint16)
    y = np.zeros((x.shape[0], H), np.float64)
    _check(lib().oracle_shared_ffn(_p(w), H, I, _p(x), x.shape[0], _p(y)), "shared_ffn")
    return y


def route(W, bias, x, k: int, score: str):
    """Returns (idx [T,k] int32 in selection order, w [T,k] fp64, z [T,E] fp64)."""
    W = _c(W, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    x = _c(np.atleast_2d(x), np.float64)
    E, H = W.shape
    T = x.shape[0]
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    z = np.zeros((T, E), np.float64)
    _check(lib().oracle_route(_p(W), _p(b), E, H, _p(x), T, k, SCORE[score], _p(idx),
                              _p(w), _p(z)), "route")
    return idx, w, z


def layer(W, bias, k: int, score: str, records: Sequence[np.ndarray], shared,
          H: int, I: int, x):
    """Returns (out [T,H] fp64, idx [T,k], w [T,k])."""
    W = _c(W, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    x = _c(np.atleast_2d(x), np.float64)
    E = W.shape[0]
    T = x.shape[0]
    recs = [_c(r, np.uint8) for r in records]
    ptrs = (ctypes.c_void_p * E)(*[r.ctypes.data for r in recs])
    sh = None if shared is None else _c(shared, np.uint16)
    out = np.zeros((T, H), np.float64)
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    _check(lib().oracle_layer(_p(W), _p(b), E, k, SCORE[score], ptrs, _p(sh), H, I,
                              _p(x), T, _p(out), _p(idx), _p(w)), "layer")
    return out, idx, w


def lru(keys, capacity: int):
    """Returns (hit, slot, evicted) arrays for a key sequence."""
    keys = _c(keys, np.int64)
    n = keys.size
    hit = np.zeros(n, np.int32)
    slot = np.zeros(n, np.int32)
    ev = np.zeros(n, np.int64)
    _check(lib().oracle_lru(_p(keys), n, capacity, _p(hit), _p(slot), _p(ev)), "lru")
    return hit, slot, ev


def two_tier(keys, c1: int, c2: int):
    """Two exclusive LRU tiers (upper c1 slots, lower c2 slots) over a key
    sequence.  Returns a dict of arrays: hit1, slot1, ev1 (upper tier, as
    lru), hit2 (-1 upper hit, 0 absent below, 1 found below), slot2 (lower
    slot it was found in, -1), dslot and dev (lower slot the upper victim went
    to, key that left the lower tier for it; -1 if none)."""
    keys = _c(keys, np.int64)
    n = keys.size
    out = {"hit1": np.zeros(n, np.int32), "slot1": np.zeros(n, np.int32), "ev1": np.zeros(n, np.int64),
           "hit2": np.zeros(n, np.int32), "slot2": np.zeros(n, np.int32), "dslot": np.zeros(n, np.int32),
           "dev": np.zeros(n, np.int64)}
    _check(lib().oracle_two_tier(_p(keys), n, c1, c2, _p(out["hit1"]), _p(out["slot1"]), _p(out["ev1"]),
                                 _p(out["hit2"]), _p(out["slot2"]), _p(out["dslot"]), _p(out["dev"])), "two_tier")
    return out


def stream_trace(idx, nlayers: int, E: int, capacity: int, layer0: int = 0):
    """Cache trace for selected experts idx [steps, k] (decode order).
    Returns (key, hit, slot, evicted), each [steps * k]."""
    idx = _c(idx, np.int32)
    steps, k = idx.shape
    n = steps * k
    key = np.zeros(n, np.int64)
    hit = np.zeros(n, np.int32)
    slot = np.zeros(n, np.int32)
    ev = np.zeros(n, np.int64)
    _check(lib().oracle_stream_trace(_p(idx), steps, nlayers, layer0, E, k, capacity,
                                     _p(key), _p(hit), _p(slot), _p(ev)), "stream_trace")
    return key, hit, slot, ev
