"""ctypes binding of libmoe (include/moe.h).  Argument marshalling only: every
step of the path runs in the library's HIP kernels.  There is no fallback:
if libmoe.so is missing the import of a compute function raises."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

P = ctypes.c_void_p
I32 = ctypes.c_int32
U32 = ctypes.c_uint32
I64 = ctypes.c_int64
U64 = ctypes.c_uint64
SZ = ctypes.c_size_t

MOE_OK, MOE_E_INVAL, MOE_E_HIP, MOE_E_SPACE, MOE_E_STATE, MOE_E_NOMEM = 0, -1, -2, -3, -4, -5
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_MAX_K, MOE_MAX_E = 32, 1024
MOE_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
MOE_NO_KEY = 0xFFFFFFFF


class MoeRecordLayout(ctypes.Structure):
    _fields_ = [("offset", I64 * 9), ("size", I64 * 9), ("nbytes", I64), ("padded", I64)]


class MoeRouter(ctypes.Structure):
    _fields_ = [("weight", P), ("bias", P), ("E", I32), ("k", I32), ("score_fn", I32)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("H", I32), ("I", I32), ("router", MoeRouter), ("records", P), ("shared", P)]


class MoeTraceRec(ctypes.Structure):
    _fields_ = [("key", U32), ("hit", I32), ("slot", I32), ("evicted", U32)]


# name -> (restype, argtypes); the complete list of symbols moe.h declares
SIGNATURES = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (ctypes.c_int, []),
    "moe_hbm_read": (ctypes.c_int, [P, ctypes.c_uint64, P, P]),
    "moe_rvq_record_layout": (ctypes.c_int, [I32, I32, ctypes.POINTER(MoeRecordLayout)]),
    "moe_route_workspace_bytes": (SZ, [I32, I32]),
    "moe_route_topk": (ctypes.c_int, [ctypes.POINTER(MoeRouter), P, I32, I32, I32, P, P, P, SZ, P]),
    "moe_expert_ffn_workspace_bytes": (SZ, [I32, I32, I32]),
    "moe_expert_ffn_rvq": (ctypes.c_int, [P, I32, I32, P, I32, P, P, I32, P, SZ, P]),
    "moe_layer_workspace_bytes": (SZ, [ctypes.POINTER(MoeLayer), I32]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(MoeLayer), P, I32, I32, P, P, P, P, SZ, P]),
    "moe_decode_workspace_bytes": (SZ, [ctypes.POINTER(MoeLayer), I32]),
    "moe_decode_forward": (ctypes.c_int, [ctypes.POINTER(MoeLayer), I32, P, I32, P, P, P, SZ, P]),
    "moe_decode_status": (ctypes.c_int, [P, ctypes.POINTER(I32)]),
    "moe_decode_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeLayer), I32, P, I32, P, P, P]),
    "moe_decode_gate_up_method": (ctypes.c_int, [P, I32, ctypes.POINTER(I32)]),
    "moe_decode_down_method": (ctypes.c_int, [P, I32, ctypes.POINTER(I32)]),
    "moe_grouped_workspace_bytes": (SZ, [ctypes.POINTER(MoeLayer), I32]),
    "moe_layer_forward_grouped": (ctypes.c_int, [ctypes.POINTER(MoeLayer), P, I32, I32, P, P, P, P, SZ, P]),
    "expert_cache_create": (ctypes.c_int, [I32, U64, P, ctypes.POINTER(P)]),
    "expert_cache_destroy": (None, [P]),
    "expert_cache_lookup": (ctypes.c_int, [P, U32, ctypes.POINTER(I32)]),
    "expert_cache_insert": (ctypes.c_int, [P, U32, P, P, ctypes.POINTER(I32), ctypes.POINTER(U32)]),
    "expert_cache_wait": (ctypes.c_int, [P, I32, P]),
    "expert_cache_release": (ctypes.c_int, [P, I32, P]),
    "expert_cache_slot_ptr": (ctypes.c_int, [P, I32, ctypes.POINTER(P)]),
    "expert_cache_trace": (ctypes.c_int, [P, ctypes.POINTER(MoeTraceRec), I64, ctypes.POINTER(I64)]),
    "expert_cache_trace_reset": (ctypes.c_int, [P]),
    "expert_cache_stats": (ctypes.c_int, [P, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                          ctypes.POINTER(I64), ctypes.POINTER(I64)]),
    "moe_lru_stack_distances": (ctypes.c_int, [P, I64, P]),
    "expert_cache_stats_ahead": (ctypes.c_int, [P, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                                ctypes.POINTER(I64), ctypes.POINTER(I64)]),
    "moe_host_tier_create": (ctypes.c_int, [ctypes.c_char_p, U64, I64, I32, P, I32, ctypes.POINTER(P)]),
    "moe_host_tier_create_exclusive": (ctypes.c_int, [ctypes.c_char_p, U64, I64, I32, P, I32, ctypes.POINTER(P)]),
    "moe_host_tier_demotions": (ctypes.c_int, [P, ctypes.POINTER(I64)]),
    "moe_host_tier_destroy": (None, [P]),
    "moe_host_tier_stats": (ctypes.c_int, [P, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64),
                                           ctypes.POINTER(I64), ctypes.POINTER(I64)]),
    "moe_host_tier_trace": (ctypes.c_int, [P, ctypes.POINTER(MoeTraceRec), I64, ctypes.POINTER(I64)]),
    "moe_layer_forward_streamed_tiered": (ctypes.c_int, [ctypes.POINTER(MoeLayer), P, U32, P, I64, P, I32, P, P, P,
                                                         SZ, P, P]),
    "moe_layer_forward_streamed_ahead": (ctypes.c_int, [ctypes.POINTER(MoeLayer), P, U32, P, P, I32, P, P,
                                                        P, SZ, P, P, ctypes.POINTER(MoeLayer), U32, P, I32,
                                                        ctypes.c_float]),
    "moe_streamed_workspace_bytes": (SZ, [ctypes.POINTER(MoeLayer), I32]),
    "moe_layer_forward_streamed": (ctypes.c_int, [ctypes.POINTER(MoeLayer), P, U32, P, P, I32, P, P,
                                                  P, SZ, P, P]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run routed_expert_streaming_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(rc: int, fn: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, fn, lib().moe_last_error().decode(errors="replace"))
