"""MI355X-native routed-expert MoE decode path.

Python face of libmoe (include/moe.h): torch supplies device memory and
streams; every computation runs in the library's HIP kernels.  Names follow
the C ABI: route_topk, expert_ffn_rvq, layer_forward, decode_forward,
layer_forward_grouped, ExpertCache (expert_cache_*), layer_forward_streamed,
decode_forward_noalloc,
lru_stack_distances, HostTier (moe_host_tier_*), hbm_read.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import (MOE_DTYPE_BF16, MOE_DTYPE_F32, MOE_E_INVAL, MOE_MAX_K, MOE_NO_KEY, MOE_SCORE_SIGMOID,
                   MOE_SCORE_SOFTMAX, MoeError, MoeLayer, MoeRecordLayout, MoeRouter,
                   MoeTraceRec, check, lib)

SCORE = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return MOE_DTYPE_F32
    if x.dtype == torch.bfloat16:
        return MOE_DTYPE_BF16
    raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def abi_version() -> int:
    return lib().moe_abi_version()


HBM_READ_BLOCKS = 2048   # MOE_HBM_READ_BLOCKS


def hbm_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One plain streaming read of buf's bytes (moe_hbm_read, the reference
    rate for expert-weight bandwidth).  Returns the [HBM_READ_BLOCKS] int32
    partials, whose XOR equals the XOR of buf's 32-bit words."""
    _need(buf.is_contiguous(), "buf must be contiguous")
    if sink is None:
        sink = torch.empty(HBM_READ_BLOCKS, dtype=torch.int32, device=buf.device)
    _need(sink.numel() >= HBM_READ_BLOCKS and sink.dtype == torch.int32, "sink must hold HBM_READ_BLOCKS int32")
    nbytes = buf.numel() * buf.element_size()
    check(lib().moe_hbm_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "moe_hbm_read")
    return sink


def rvq_record_layout(H: int, I: int) -> MoeRecordLayout:
    out = MoeRecordLayout()
    check(lib().moe_rvq_record_layout(H, I, ctypes.byref(out)), "moe_rvq_record_layout")
    return out


# ------------------------------------------------------------------ layers
@dataclass
class Router:
    weight: torch.Tensor                 # [E, H] fp32 device
    k: int
    score: str = "softmax"
    bias: Optional[torch.Tensor] = None  # [E] fp32 device

    def struct(self) -> MoeRouter:
        E = self.weight.shape[0]
        return MoeRouter(self.weight.data_ptr(), None if self.bias is None else self.bias.data_ptr(),
                         E, self.k, SCORE[self.score])


@dataclass
class Layer:
    """One MoE layer: router, expert records resident in HBM (any device
    tensors, 256-byte aligned), optional dense bf16 shared expert."""
    H: int
    I: int
    router: Router
    records: Sequence[torch.Tensor] = ()            # E uint8 device tensors (resident path)
    shared: Optional[torch.Tensor] = None           # bf16/int16 device tensor, 3*H*I elements
    record_ptrs: Optional[torch.Tensor] = field(default=None, repr=False)

    def __post_init__(self):
        if self.records and self.record_ptrs is None:
            self.set_records(self.records)

    def set_records(self, records: Sequence[torch.Tensor] = (), ptrs: Optional[Sequence[int]] = None):
        if ptrs is None:
            ptrs = [r.data_ptr() for r in records]
        self.records = records
        dev = self.router.weight.device
        self.record_ptrs = torch.tensor(list(ptrs), dtype=torch.int64).to(dev)

    def struct(self) -> MoeLayer:
        return MoeLayer(self.H, self.I, self.router.struct(),
                        None if self.record_ptrs is None else self.record_ptrs.data_ptr(),
                        None if self.shared is None else self.shared.data_ptr())


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ routing
def route_topk(router: Router, x: torch.Tensor, stream=None, ws: Optional[torch.Tensor] = None):
    """idx [T, k] int32 and w [T, k] fp32 for x [T, H] (fp32 or bf16)."""
    _need(x.dim() == 2 and x.is_contiguous(), "x must be a contiguous [T, H] tensor")
    T, H = x.shape
    E = router.weight.shape[0]
    idx = torch.empty((T, router.k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, router.k), dtype=torch.float32, device=x.device)
    need = lib().moe_route_workspace_bytes(E, T)
    ws = ws if ws is not None else _ws(need, x.device)
    r = router.struct()
    check(lib().moe_route_topk(ctypes.byref(r), _ptr(x), _dtype_code(x), T, H, _ptr(idx), _ptr(w),
                               _ptr(ws), ws.numel(), _stream(stream)), "moe_route_topk")
    return idx, w


# --------------------------------------------------------------- expert FFN
def expert_ffn_rvq(record: torch.Tensor, H: int, I: int, x: torch.Tensor,
                   gate_w: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                   accumulate: bool = False, stream=None, ws: Optional[torch.Tensor] = None):
    """y [T, H] (+)= gate_w[t] * expert(x_t) for one RVQ expert record."""
    _need(x.dim() == 2 and x.dtype == torch.float32 and x.is_contiguous(), "x must be contiguous fp32 [T, H]")
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
        accumulate = False
    need = lib().moe_expert_ffn_workspace_bytes(H, I, T)
    ws = ws if ws is not None else _ws(need, x.device)
    check(lib().moe_expert_ffn_rvq(_ptr(record), H, I, _ptr(x), T, _ptr(gate_w), _ptr(y), int(accumulate),
                                   _ptr(ws), ws.numel(), _stream(stream)), "moe_expert_ffn_rvq")
    return y


# ------------------------------------------------------------------- layer
def layer_workspace_bytes(layer: Layer, T: int) -> int:
    s = layer.struct()
    return lib().moe_layer_workspace_bytes(ctypes.byref(s), T)


def layer_forward(layer: Layer, x: torch.Tensor, stream=None, ws: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, want_routing: bool = True):
    """out [T, H] fp32, idx [T, k], w [T, k] for x [T, H] (fp32 or bf16)."""
    _need(x.dim() == 2 and x.is_contiguous(), "x must be a contiguous [T, H] tensor")
    T = x.shape[0]
    k = layer.router.k
    out = out if out is not None else torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if want_routing else None
    w = torch.empty((T, k), dtype=torch.float32, device=x.device) if want_routing else None
    s = layer.struct()
    need = lib().moe_layer_workspace_bytes(ctypes.byref(s), T)
    ws = ws if ws is not None else _ws(need, x.device)
    check(lib().moe_layer_forward(ctypes.byref(s), _ptr(x), _dtype_code(x), T, _ptr(out), _ptr(idx), _ptr(w),
                                  _ptr(ws), ws.numel(), _stream(stream)), "moe_layer_forward")
    return out, idx, w


def _layer_array(layers: Sequence[Layer]):
    arr = (MoeLayer * len(layers))()
    for i, l in enumerate(layers):
        arr[i] = l.struct()
    return arr


def decode_workspace_bytes(layers: Sequence[Layer]) -> int:
    arr = _layer_array(layers)
    n = lib().moe_decode_workspace_bytes(arr, len(layers))
    if n == 0:
        raise MoeError(MOE_E_INVAL, "moe_decode_workspace_bytes", lib().moe_last_error().decode(errors="replace"))
    return n


def decode_forward(layers: Sequence[Layer], x: torch.Tensor, stream=None, ws: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None, want_idx: bool = True):
    """x [T, L, H] fp32 -> out [T, L, H] fp32, idx [T, L, k] (token-major decode)."""
    _need(x.dim() == 3 and x.dtype == torch.float32 and x.is_contiguous(), "x must be contiguous fp32 [T, L, H]")
    T, nL, H = x.shape
    _need(nL == len(layers), "x's layer dimension must match len(layers)")
    arr = _layer_array(layers)
    k = layers[0].router.k
    out = out if out is not None else torch.empty_like(x)
    if want_idx and idx is None:
        idx = torch.empty((T, nL, k), dtype=torch.int32, device=x.device)
    need = lib().moe_decode_workspace_bytes(arr, nL)
    ws = ws if ws is not None else _ws(need, x.device)
    check(lib().moe_decode_forward(arr, nL, _ptr(x), T, _ptr(out), _ptr(idx if want_idx else None),
                                   _ptr(ws), ws.numel(), _stream(stream)), "moe_decode_forward")
    return out, (idx if want_idx else None)


def decode_gate_up_method(layers: Sequence[Layer]) -> str:
    """"lookup" or "gathers": the gate/up method decode_forward uses for
    these layers on the current device."""
    arr = _layer_array(layers)
    m = ctypes.c_int32()
    check(lib().moe_decode_gate_up_method(arr, len(layers), ctypes.byref(m)), "moe_decode_gate_up_method")
    return "lookup" if m.value else "gathers"


def decode_down_method(layers: Sequence[Layer]) -> str:
    """"lookup" or "gathers": the down method decode_forward uses for these
    layers on the current device."""
    arr = _layer_array(layers)
    m = ctypes.c_int32()
    check(lib().moe_decode_down_method(arr, len(layers), ctypes.byref(m)), "moe_decode_down_method")
    return "lookup" if m.value else "gathers"


NOALLOC_SCRATCH_BYTES = _lib.MOE_NOALLOC_SCRATCH_BYTES


def decode_forward_noalloc(layers: Sequence[Layer], x: torch.Tensor, stream=None,
                           out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                           want_idx: bool = True):
    """decode_forward with the library's own device scratch array as the
    workspace (moe_decode_forward_noalloc: nothing is allocated by the
    library; calls that overlap on one device race)."""
    _need(x.dim() == 3 and x.dtype == torch.float32 and x.is_contiguous(), "x must be contiguous fp32 [T, L, H]")
    T, nL, H = x.shape
    _need(nL == len(layers), "x's layer dimension must match len(layers)")
    arr = _layer_array(layers)
    k = layers[0].router.k
    out = out if out is not None else torch.empty_like(x)
    if want_idx and idx is None:
        idx = torch.empty((T, nL, k), dtype=torch.int32, device=x.device)
    check(lib().moe_decode_forward_noalloc(arr, nL, _ptr(x), T, _ptr(out), _ptr(idx if want_idx else None),
                                           _stream(stream)), "moe_decode_forward_noalloc")
    return out, (idx if want_idx else None)


def decode_status(ws: Optional[torch.Tensor]) -> bool:
    """True if any decode_forward on this workspace (ws = None: any
    decode_forward_noalloc on the current device) since the previous call hit
    its device-side wait limit (those outputs are invalid); resets the
    status.  Synchronises."""
    flag = ctypes.c_int32()
    check(lib().moe_decode_status(_ptr(ws), ctypes.byref(flag)), "moe_decode_status")
    return bool(flag.value)


def grouped_workspace_bytes(layer: Layer, T: int) -> int:
    s = layer.struct()
    return lib().moe_grouped_workspace_bytes(ctypes.byref(s), T)


def layer_forward_grouped(layer: Layer, x: torch.Tensor, stream=None, ws: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None):
    """Batched layer on matrix cores: out [T, H] fp32, idx [T, k], w [T, k]."""
    _need(x.dim() == 2 and x.is_contiguous(), "x must be a contiguous [T, H] tensor")
    T = x.shape[0]
    k = layer.router.k
    out = out if out is not None else torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    s = layer.struct()
    need = lib().moe_grouped_workspace_bytes(ctypes.byref(s), T)
    ws = ws if ws is not None else _ws(need, x.device)
    check(lib().moe_layer_forward_grouped(ctypes.byref(s), _ptr(x), _dtype_code(x), T, _ptr(out), _ptr(idx),
                                          _ptr(w), _ptr(ws), ws.numel(), _stream(stream)),
          "moe_layer_forward_grouped")
    return out, idx, w


# ------------------------------------------------------------------- cache
class ExpertCache:
    """HBM expert-slot LRU cache over a caller-owned device pool."""

    def __init__(self, capacity: int, slot_bytes: int, pool: torch.Tensor):
        _need(pool.numel() * pool.element_size() >= capacity * slot_bytes, "pool too small")
        self.capacity, self.slot_bytes, self.pool = capacity, slot_bytes, pool
        h = ctypes.c_void_p()
        check(lib().expert_cache_create(capacity, slot_bytes, _ptr(pool), ctypes.byref(h)), "expert_cache_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib().expert_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup(self, key: int) -> int:
        slot = ctypes.c_int32()
        check(lib().expert_cache_lookup(self.handle, key, ctypes.byref(slot)), "expert_cache_lookup")
        return slot.value

    def insert(self, key: int, host_src: int, copy_stream=None):
        slot, ev = ctypes.c_int32(), ctypes.c_uint32()
        check(lib().expert_cache_insert(self.handle, key, ctypes.c_void_p(host_src), _stream(copy_stream),
                                        ctypes.byref(slot), ctypes.byref(ev)), "expert_cache_insert")
        return slot.value, (None if ev.value == MOE_NO_KEY else ev.value)

    def wait(self, slot: int, stream=None):
        check(lib().expert_cache_wait(self.handle, slot, _stream(stream)), "expert_cache_wait")

    def release(self, slot: int, stream=None):
        check(lib().expert_cache_release(self.handle, slot, _stream(stream)), "expert_cache_release")

    def slot_ptr(self, slot: int) -> int:
        p = ctypes.c_void_p()
        check(lib().expert_cache_slot_ptr(self.handle, slot, ctypes.byref(p)), "expert_cache_slot_ptr")
        return p.value

    def trace(self):
        """List of (key, hit, slot, evicted or None)."""
        n = ctypes.c_int64()
        lib().expert_cache_trace(self.handle, None, 0, ctypes.byref(n))
        buf = (MoeTraceRec * max(n.value, 1))()
        check(lib().expert_cache_trace(self.handle, buf, n.value, ctypes.byref(n)), "expert_cache_trace")
        return [(r.key, r.hit, r.slot, None if r.evicted == MOE_NO_KEY else r.evicted) for r in buf[:n.value]]

    def trace_reset(self):
        check(lib().expert_cache_trace_reset(self.handle), "expert_cache_trace_reset")

    def stats(self):
        v = [ctypes.c_int64() for _ in range(8)]
        check(lib().expert_cache_stats(self.handle, *[ctypes.byref(x) for x in v[:4]]), "expert_cache_stats")
        check(lib().expert_cache_stats_ahead(self.handle, *[ctypes.byref(x) for x in v[4:]]),
              "expert_cache_stats_ahead")
        return dict(zip(("lookups", "hits", "inserts", "evictions", "ahead_inserted", "ahead_present",
                         "ahead_used", "ahead_wasted"), [x.value for x in v]))


def lru_stack_distances(keys) -> "numpy.ndarray":
    """LRU stack distance of each reference in a sequence of cache keys
    (moe_lru_stack_distances): -1 at a first reference, else the number of
    distinct keys referenced since the previous reference to the same key."""
    import numpy as np
    k = np.ascontiguousarray(keys, dtype=np.uint32)
    d = np.empty(k.shape[0], dtype=np.int32)
    check(lib().moe_lru_stack_distances(k.ctypes.data if k.size else None, k.shape[0],
                                        d.ctypes.data if d.size else None), "moe_lru_stack_distances")
    return d


def lru_hits_at(dist, capacities: Sequence[int]) -> List[int]:
    """Hits of an LRU cache of each capacity, started empty, on the reference
    string whose stack distances are dist (a reference hits iff 0 <= d < C)."""
    import numpy as np
    d = np.asarray(dist)
    warm = np.sort(d[d >= 0])
    return [int(np.searchsorted(warm, c, side="left")) for c in capacities]


class HostTier:
    """Expert records in a file (moe_host_tier_*): O_DIRECT reads into a
    pinned pool of `slots` records kept as LRU, the source of the HBM
    cache's misses in layer_forward_streamed(..., tier=(this, record0)).
    exclusive=True makes it the HBM cache's exclusive lower tier
    (moe_host_tier_create_exclusive): it holds the HBM cache's evicted
    records, slots - MOE_MAX_K of them, and the pool has MOE_MAX_K more
    pages for records in transit."""

    def __init__(self, path: str, record_bytes: int, n_records: int, slots: int, io_threads: int = 8,
                 exclusive: bool = False):
        self.pool = torch.empty(slots * record_bytes + 4096, dtype=torch.uint8, pin_memory=True)
        base = (self.pool.data_ptr() + 4095) & ~4095
        h = ctypes.c_void_p()
        fn = lib().moe_host_tier_create_exclusive if exclusive else lib().moe_host_tier_create
        check(fn(path.encode(), record_bytes, n_records, slots, base, io_threads, ctypes.byref(h)),
              "moe_host_tier_create_exclusive" if exclusive else "moe_host_tier_create")
        self.handle = h
        self.exclusive = exclusive

    def close(self):
        if self.handle:
            lib().moe_host_tier_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stats(self):
        v = [ctypes.c_int64() for _ in range(5)]
        check(lib().moe_host_tier_stats(self.handle, *[ctypes.byref(x) for x in v]), "moe_host_tier_stats")
        d = dict(zip(("lookups", "hits", "reads", "read_bytes", "read_ns"), [x.value for x in v]))
        dm = ctypes.c_int64()
        check(lib().moe_host_tier_demotions(self.handle, ctypes.byref(dm)), "moe_host_tier_demotions")
        d["demotions"] = dm.value
        return d

    def trace(self):
        """List of (key, hit, slot, evicted or None); keys are record indices."""
        n = ctypes.c_int64()
        lib().moe_host_tier_trace(self.handle, None, 0, ctypes.byref(n))
        buf = (MoeTraceRec * max(n.value, 1))()
        check(lib().moe_host_tier_trace(self.handle, buf, n.value, ctypes.byref(n)), "moe_host_tier_trace")
        return [(r.key, r.hit, r.slot, None if r.evicted == MOE_NO_KEY else r.evicted) for r in buf[:n.value]]


def streamed_workspace_bytes(layer: Layer, T: int = 1) -> int:
    s = layer.struct()
    return lib().moe_streamed_workspace_bytes(ctypes.byref(s), T)


def layer_forward_streamed(layer: Layer, cache: ExpertCache, layer_id: int, experts_host: Sequence[int],
                           x: torch.Tensor, copy_stream: torch.cuda.Stream, stream=None,
                           ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           idx: Optional[torch.Tensor] = None, host_table=None, ahead=None, tier=None):
    """One decode step of one layer fed from the slot cache.  experts_host:
    E pinned host addresses of the layer's records (or a prebuilt ctypes
    array).  ahead = (next_layer, next_layer_id, next_host_table, k_ahead[,
    min_weight]) adds the look-ahead read of moe_layer_forward_streamed_ahead
    (predictions with a smaller weight are not read ahead); tier =
    (HostTier, record0) takes the misses from the file tier instead
    (moe_layer_forward_streamed_tiered)."""
    _need(x.dim() == 2 and x.shape[0] == 1 and x.dtype == torch.float32, "x must be fp32 [1, H]")
    out = out if out is not None else torch.empty((1, layer.H), dtype=torch.float32, device=x.device)
    s = layer.struct()
    table = None
    if tier is None:
        table = host_table if host_table is not None else (ctypes.c_void_p * len(experts_host))(*experts_host)
    need = lib().moe_streamed_workspace_bytes(ctypes.byref(s), 1)
    ws = ws if ws is not None else _ws(need, x.device)
    if tier is not None:
        ht, record0 = tier
        check(lib().moe_layer_forward_streamed_tiered(ctypes.byref(s), cache.handle, layer_id, ht.handle, record0,
                                                      _ptr(x), 1, _ptr(out), _ptr(idx), _ptr(ws), ws.numel(),
                                                      _stream(stream), _stream(copy_stream)),
              "moe_layer_forward_streamed_tiered")
        return out
    if ahead is None:
        check(lib().moe_layer_forward_streamed(ctypes.byref(s), cache.handle, layer_id, table, _ptr(x), 1, _ptr(out),
                                               _ptr(idx), _ptr(ws), ws.numel(), _stream(stream),
                                               _stream(copy_stream)), "moe_layer_forward_streamed")
        return out
    nxt, nxt_id, nxt_host, k_ahead = ahead[:4]
    min_weight = float(ahead[4]) if len(ahead) > 4 else 0.0
    ns = nxt.struct()
    ntable = nxt_host if not isinstance(nxt_host, (list, tuple)) else (ctypes.c_void_p * len(nxt_host))(*nxt_host)
    check(lib().moe_layer_forward_streamed_ahead(ctypes.byref(s), cache.handle, layer_id, table, _ptr(x), 1,
                                                 _ptr(out), _ptr(idx), _ptr(ws), ws.numel(), _stream(stream),
                                                 _stream(copy_stream), ctypes.byref(ns), nxt_id, ntable, k_ahead,
                                                 min_weight),
          "moe_layer_forward_streamed_ahead")
    return out
