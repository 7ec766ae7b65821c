"""Place a synthetic workload (``synth``) in device memory as library inputs:
router weights, biases, expert records (one pool per layer), shared experts,
and the per-(token, layer) activations; or, for streamed decode, the expert
records in pinned host memory."""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

import synth

from . import Layer, Router


def _threads() -> int:
    return min(16, len(os.sched_getaffinity(0)))


class DeviceWorkload:
    """All layers of a config resident in HBM.  ``layers``/``experts`` may
    restrict what is uploaded (a reduced variant for quick tests)."""

    def __init__(self, cfg: synth.MoEConfig, device="cuda", layers: Optional[Sequence[int]] = None,
                 with_records: bool = True, batch: int = 16):
        self.cfg = cfg
        self.wl = synth.Workload(cfg)
        self.device = torch.device(device)
        self.layer_ids = list(range(cfg.layers)) if layers is None else list(layers)
        lay = self.wl.layout
        self.record_stride = lay.padded
        self.layers: List[Layer] = []
        self.pools: List[torch.Tensor] = []
        for L in self.layer_ids:
            W = torch.from_numpy(self.wl.router(L)).to(self.device)
            b = self.wl.bias(L)
            bt = None if b is None else torch.from_numpy(b).to(self.device)
            sh = self.wl.shared(L)
            sht = None if sh is None else torch.from_numpy(sh.view(np.int16)).to(self.device)
            layer = Layer(cfg.H, cfg.I, Router(W, cfg.k, cfg.score, bt), shared=sht)
            if with_records:
                pool = torch.empty(cfg.E * lay.padded, dtype=torch.uint8, device=self.device)
                self._fill_pool(L, pool, batch)
                base = pool.data_ptr()
                layer.set_records(ptrs=[base + e * lay.padded for e in range(cfg.E)])
                self.pools.append(pool)
            self.layers.append(layer)
        torch.cuda.synchronize(self.device)

    def _fill_pool(self, L: int, pool: torch.Tensor, batch: int):
        cfg, pad = self.cfg, self.wl.layout.padded
        nb = min(batch, cfg.E)
        stage = [torch.empty((nb, pad), dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        events = [None, None]
        for i, e0 in enumerate(range(0, cfg.E, nb)):
            buf = stage[i % 2]
            if events[i % 2] is not None:
                events[i % 2].synchronize()
            n = min(nb, cfg.E - e0)
            arr = buf.numpy()
            self.wl.fill_records([(L, e0 + j) for j in range(n)], [arr[j] for j in range(n)], _threads())
            pool[e0 * pad:(e0 + n) * pad].copy_(buf[:n].reshape(-1), non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            events[i % 2] = ev
        torch.cuda.synchronize(self.device)

    def inputs(self) -> torch.Tensor:
        """x [T, L, H] fp32 (decode) or [T, H] (batched; bf16 values) on device,
        restricted to the uploaded layers."""
        x = self.wl.inputs()
        if not self.cfg.batched:
            x = x[:, self.layer_ids, :]
        return torch.from_numpy(np.ascontiguousarray(x)).to(self.device)


def write_record_file(cfg: synth.MoEConfig, path: str, layers: Sequence[int], batch: int = 64,
                      progress=None) -> int:
    """Write the records of `layers` (all E experts each) to `path`, record
    (i, e) of the i-th listed layer at index i * E + e, each padded to the
    4 KiB record stride (the file tier's layout).  Returns the stride.
    progress(records_written) is called after every batch if given."""
    wl = synth.Workload(cfg)
    stride = wl.layout.padded
    keys = [(L, e) for L in layers for e in range(cfg.E)]
    buf = np.zeros((min(batch, len(keys)), stride), dtype=np.uint8)
    with open(path, "wb") as f:
        for k0 in range(0, len(keys), batch):
            ck = keys[k0:k0 + batch]
            buf[:len(ck)] = 0
            wl.fill_records(ck, [buf[j] for j in range(len(ck))], _threads())
            f.write(buf[:len(ck)].tobytes())
            if progress:
                progress(k0 + len(ck))
    return stride


def chain_next_input(h: torch.Tensor, out: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """Chained (pre-norm) decode inputs, a stand-in for the trunk between MoE
    layers, which is not modelled: the residual stream h [H] takes the layer's
    output (h += out), and the next layer reads h rescaled to rms `scale`
    (the seeded first input's rms).  Device tensor ops on the current stream."""
    h.add_(out.reshape(h.shape))
    return (h * (scale * torch.rsqrt(h.pow(2).mean()))).reshape(1, -1)


class HostRecordPool:
    """Expert records of several layers in host memory (the cold tier of
    streamed decode): page-locked chunks of at most ``chunk_bytes`` up to
    ``pin_limit`` bytes in total, the remainder (if any) in pageable memory.
    ``pinned_records`` says how many records are page-locked.  Records are
    laid out expert-major (expert e of every layer, then e + 1), so a pin
    budget below the whole pool leaves every layer the same share of
    page-locked records (expert ids carry no popularity order): each layer's
    misses then mostly include page-locked ones, whose transfers run while
    the host stages the pageable ones.  Layer-major order would leave whole
    layers pageable, whose first miss waits for its staging."""

    def __init__(self, cfg: synth.MoEConfig, layers: Sequence[int], experts: Optional[int] = None,
                 chunk_bytes: int = 4 << 30, pin_limit: int = 52 << 30):
        self.cfg = cfg
        wl = synth.Workload(cfg)
        self.stride = wl.layout.padded
        E = cfg.E if experts is None else experts
        per_chunk = max(1, chunk_bytes // self.stride)
        keys = [(L, e) for e in range(E) for L in layers]
        self.chunks: List = []
        self.addr = {}
        self.pinned_records = 0
        pinned_bytes = 0
        for c0 in range(0, len(keys), per_chunk):
            ck = keys[c0:c0 + per_chunk]
            nbytes = len(ck) * self.stride
            t = None
            if pinned_bytes + nbytes <= pin_limit:
                try:
                    t = torch.empty((len(ck), self.stride), dtype=torch.uint8, pin_memory=True)
                    pinned_bytes += nbytes
                    self.pinned_records += len(ck)
                except Exception:             # page-locked memory exhausted
                    t = None
            if t is None:
                t = torch.empty((len(ck), self.stride), dtype=torch.uint8)
            arr = t.numpy()
            wl.fill_records(ck, [arr[j] for j in range(len(ck))], _threads())
            base = t.data_ptr()
            for j, key in enumerate(ck):
                self.addr[key] = base + j * self.stride
            self.chunks.append(t)
        self.layers = list(layers)
        self.E = E

    def table(self, L: int):
        """ctypes array of the E host record addresses of layer L."""
        return (ctypes.c_void_p * self.cfg.E)(*[self.addr.get((L, e), 0) for e in range(self.cfg.E)])
