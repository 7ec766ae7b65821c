"""Seeded synthetic workloads for the routed-expert MoE decode path.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``routed_expert_streaming_amd``).  It generates *inputs only*: router
weights, popularity biases, expert records (RVQ codes, scales, codebooks),
dense shared-expert records and token activations.  It computes none of the
method's results: no routing weights, no decoded weights, no FFN outputs.

The one place where it evaluates router logits is the workload's selection
filter (:func:`topk_margins`): the workloads are defined as "redraw until the
gap between the k-th and (k+1)-th largest logit is at least 1e-3", so that
the selected expert set is unambiguous in fp32 as well as in fp64.  The
filter only rejects draws; nothing either side produces is compared against a
value computed here.

Sources (pages on routed expert streaming):
  * "2.78조 파라미터 모델을 노트북에서: NVMe 스트리밍 추론 엔진 WASTE"
    (ttj.ttj.kr), section "유휴 가중치는 메모리가 아니라 제때 닿기만 하면
    된다": one expert = one 4 KiB-aligned record with gate, up and down
    adjacent; experts stored as residual vector quantisation at 3.00 bits per
    weight and never expanded.
  * "WARP 소개" (discuss.pytorch.kr), section "WARP의 캐시 설정에서 드러나는
    역설": the number of experts per token is a container-manifest field.
The exact shapes (groups of 8 input-dim weights, two 12-bit indices into a
per-matrix 4096x8 fp16 codebook, per-row fp16 scale) are the workload
definitions below; the pages fix only the 3.00 bit/weight budget.

Record format (this project's own; the pages say the container format is not
fixed):

  section 0  gate codes   [I rows, H cols]   3 bytes per group of 8 weights
  section 1  up codes     [I rows, H cols]
  section 2  down codes   [H rows, I cols]
  section 3  gate scales  fp16 [I]
  section 4  up scales    fp16 [I]
  section 5  down scales  fp16 [H]
  section 6  gate codebook fp16 [4096][8]
  section 7  up codebook   fp16 [4096][8]
  section 8  down codebook fp16 [4096][8]

Each section starts on a 256-byte boundary and the record is padded to 4 KiB.
A code pair for row r, group q (weights 8q..8q+7 of that row) is the 24-bit
little-endian value v = a | b << 12 (a = stage-1 index, b = stage-2 index).
Codes are stored in tiles of 64 rows x 128 columns (16 groups): the tile for
row block t and column block j starts at byte (t * (K/128) + j) * 3072 of the
section; inside it, byte p (0..47) of the 48-byte strip of row 64t + l lies
at offset (p // 16) * 1024 + l * 16 + (p % 16), and strip byte 3g + m is byte
m of group 16j + g's 24-bit value.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

CODEBOOK_ROWS = 4096
GROUP = 8
TILE_ROWS = 64
TILE_COLS = 128
STRIP_BYTES = 48           # 16 groups x 3 bytes
TILE_BYTES = TILE_ROWS * STRIP_BYTES
SECTION_ALIGN = 256
RECORD_ALIGN = 4096
MARGIN = 1e-3

# stream tags for SeedSequence spawn keys (fixed order: router, bias
# permutation, codebooks, scales, codes, shared, inputs, redraws)
TAG_ROUTER, TAG_PERM, TAG_CODEBOOK, TAG_SCALES, TAG_CODES, TAG_SHARED, \
    TAG_INPUT, TAG_REDRAW = range(1, 9)


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    layers: int
    H: int
    I: int
    E: int
    k: int
    score: str            # "softmax" | "sigmoid"
    shared: bool          # one always-on dense bf16 expert per layer
    tokens: int
    zipf: bool            # per-layer Zipf(s=1.1) popularity bias in the logits
    x_dtype: str          # "f32" | "bf16"
    batched: bool         # all tokens through one layer call (grouped path)
    cache_frac: Optional[float]   # HBM slot cache capacity / total experts
    redraw_router: bool   # margin filter redraws W (Tiny) instead of x
    seed: int

    @property
    def cache_capacity(self) -> int:
        assert self.cache_frac is not None
        return int(math.floor(self.cache_frac * self.layers * self.E))

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    # 1 layer, hidden 256, intermediate 512, 8 experts, softmax top-2, 4 tokens
    "tiny": MoEConfig("tiny", 1, 256, 512, 8, 2, "softmax", False, 4, False,
                      "f32", False, None, True, 1000),
    # Mixtral-8x7B-shaped decode: 32 layers x 8 experts, top-2, 64 tokens
    "mixtral": MoEConfig("mixtral", 32, 4096, 14336, 8, 2, "softmax", False,
                         64, False, "f32", False, None, False, 1001),
    # Kimi-Linear-48B-class decode: 27 layers x 256 experts + shared, top-8
    "kimi_linear": MoEConfig("kimi_linear", 27, 2304, 1024, 256, 8, "sigmoid",
                             True, 128, True, "f32", False, None, False, 1002),
    # batched 256-token layer: 384 experts, top-16 + shared, bf16 tokens
    "batched": MoEConfig("batched", 1, 5120, 2048, 384, 16, "sigmoid", True,
                         256, False, "bf16", True, None, False, 1003),
    # K3-scale streaming slice: 8 layers x 768 experts + shared, top-16,
    # 25% HBM slot cache, 256 tokens
    "k3_slice": MoEConfig("k3_slice", 8, 5120, 2048, 768, 16, "sigmoid", True,
                          256, True, "f32", False, 0.25, False, 1004),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


# --------------------------------------------------------------------------
# record layout (format only)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class RecordLayout:
    H: int
    I: int
    offsets: Tuple[int, ...]   # 9 section offsets
    sizes: Tuple[int, ...]     # 9 section sizes
    nbytes: int                # end of the last section (unpadded)
    padded: int                # rounded up to 4 KiB


def _align(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def record_layout(H: int, I: int) -> RecordLayout:
    if H % TILE_COLS or I % TILE_COLS:
        raise ValueError("H and I must be multiples of 128")
    code_gu = I * (H // GROUP) * 3
    code_d = H * (I // GROUP) * 3
    cb = CODEBOOK_ROWS * GROUP * 2
    sizes = (code_gu, code_gu, code_d, 2 * I, 2 * I, 2 * H, cb, cb, cb)
    offs, pos = [], 0
    for s in sizes:
        pos = _align(pos, SECTION_ALIGN)
        offs.append(pos)
        pos += s
    return RecordLayout(H, I, tuple(offs), sizes, pos, _align(pos, RECORD_ALIGN))


def shared_record_bytes(H: int, I: int) -> int:
    """Dense bf16 shared expert: gate [I,H] | up [I,H] | down [H,I]."""
    return 3 * H * I * 2


def pack_codes(v: np.ndarray) -> np.ndarray:
    """Pack 24-bit code pairs v [N, K/8] (uint32) into the tiled byte layout."""
    v = np.asarray(v, dtype=np.uint32)
    N, G = v.shape
    K = G * GROUP
    assert N % TILE_ROWS == 0 and K % TILE_COLS == 0
    b = np.stack([(v >> (8 * m)) & 0xFF for m in range(3)], axis=-1).astype(np.uint8)
    # strips: [N, K/128, 48]
    strips = b.reshape(N, K // TILE_COLS, STRIP_BYTES)
    # -> [N/64, 64, K/128, 3, 16] -> [N/64, K/128, 3, 64, 16]
    s = strips.reshape(N // TILE_ROWS, TILE_ROWS, K // TILE_COLS, 3, 16)
    return np.ascontiguousarray(s.transpose(0, 2, 3, 1, 4)).reshape(-1)


def unpack_codes(buf: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of :func:`pack_codes` (format only): bytes -> v [N, K/8]."""
    s = np.asarray(buf, dtype=np.uint8)[: N * K * 3 // GROUP]
    s = s.reshape(N // TILE_ROWS, K // TILE_COLS, 3, TILE_ROWS, 16)
    strips = s.transpose(0, 3, 1, 2, 4).reshape(N, K // GROUP, 3).astype(np.uint32)
    return strips[..., 0] | (strips[..., 1] << 8) | (strips[..., 2] << 16)


def split_pair(v: np.ndarray):
    v = np.asarray(v, dtype=np.uint32)
    return v & 0xFFF, v >> 12


# --------------------------------------------------------------------------
# value conversions used for generation
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (f >> 16) & 1
    r = (f + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------
def rng_for(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n]


def gen_codebooks(seed: int, layer: int, expert: int) -> np.ndarray:
    """3 codebooks [3, 4096, 8] fp16, values N(0,1)/sqrt(2) rounded to fp16."""
    rng = rng_for(seed, TAG_CODEBOOK, layer, expert)
    return (rng.standard_normal((3, CODEBOOK_ROWS, GROUP)) / math.sqrt(2.0)).astype(np.float16)


def gen_scales(seed: int, layer: int, expert: int, H: int, I: int):
    """Per-row fp16 scales U(0.01, 0.03) for gate [I], up [I], down [H]."""
    rng = rng_for(seed, TAG_SCALES, layer, expert)
    s = rng.uniform(0.01, 0.03, 2 * I + H).astype(np.float16)
    return s[:I], s[I:2 * I], s[2 * I:]


def fill_record(buf: np.ndarray, cfg: MoEConfig, layer: int, expert: int) -> None:
    """Write expert (layer, expert)'s record into ``buf`` (uint8, >= padded)."""
    lay = record_layout(cfg.H, cfg.I)
    buf[: lay.padded] = 0
    rng = rng_for(cfg.seed, TAG_CODES, layer, expert)
    ncode = lay.offsets[2] + lay.sizes[2]    # the three code sections are contiguous
    assert lay.offsets[1] == lay.sizes[0] and lay.offsets[2] == 2 * lay.sizes[0]
    buf[:ncode] = random_bytes(rng, ncode)
    sg, su, sd = gen_scales(cfg.seed, layer, expert, cfg.H, cfg.I)
    for sec, arr in ((3, sg), (4, su), (5, sd)):
        buf[lay.offsets[sec]: lay.offsets[sec] + lay.sizes[sec]] = arr.view(np.uint8)
    cbs = gen_codebooks(cfg.seed, layer, expert)
    for m in range(3):
        o = lay.offsets[6 + m]
        buf[o: o + lay.sizes[6 + m]] = cbs[m].reshape(-1).view(np.uint8)


def make_record(cfg: MoEConfig, layer: int, expert: int) -> np.ndarray:
    lay = record_layout(cfg.H, cfg.I)
    buf = np.empty(lay.padded, dtype=np.uint8)
    fill_record(buf, cfg, layer, expert)
    return buf


def build_record(H: int, I: int, gate_codes, up_codes, down_codes,
                 scales, codebooks) -> np.ndarray:
    """Assemble a record from explicit parts (used by tests that construct
    special cases).  ``*_codes`` are 24-bit code pairs [rows, cols/8];
    ``scales`` = (gate [I], up [I], down [H]) fp16; ``codebooks`` [3,4096,8] fp16."""
    lay = record_layout(H, I)
    buf = np.zeros(lay.padded, dtype=np.uint8)
    for sec, (v, n, kk) in enumerate(((gate_codes, I, H), (up_codes, I, H), (down_codes, H, I))):
        p = pack_codes(np.asarray(v).reshape(n, kk // GROUP))
        buf[lay.offsets[sec]: lay.offsets[sec] + p.size] = p
    for sec, arr in zip((3, 4, 5), scales):
        a = np.asarray(arr, dtype=np.float16)
        buf[lay.offsets[sec]: lay.offsets[sec] + a.nbytes] = a.view(np.uint8)
    cbs = np.asarray(codebooks, dtype=np.float16)
    for m in range(3):
        o = lay.offsets[6 + m]
        buf[o: o + lay.sizes[6 + m]] = cbs[m].reshape(-1).view(np.uint8)
    return buf


def record_parts(buf: np.ndarray, H: int, I: int):
    """Read a record back into parts (format only; no decoding of weights)."""
    lay = record_layout(H, I)
    o = lay.offsets
    codes = [unpack_codes(buf[o[0]:], I, H), unpack_codes(buf[o[1]:], I, H),
             unpack_codes(buf[o[2]:], H, I)]
    sc = [buf[o[s]: o[s] + lay.sizes[s]].view(np.float16) for s in (3, 4, 5)]
    cbs = [buf[o[s]: o[s] + lay.sizes[s]].view(np.float16).reshape(CODEBOOK_ROWS, GROUP)
           for s in (6, 7, 8)]
    return codes, sc, cbs


def make_shared(cfg: MoEConfig, layer: int) -> np.ndarray:
    """Dense bf16 shared expert gate [I,H] | up [I,H] | down [H,I] as uint16 bits,
    values N(0, 0.02^2)."""
    rng = rng_for(cfg.seed, TAG_SHARED, layer)
    n = 3 * cfg.H * cfg.I
    w = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
    return to_bf16_bits(w)


def make_router(cfg: MoEConfig, layer: int, attempt: int = 0) -> np.ndarray:
    """Router weights [E, H] fp32, N(0, 0.05^2)."""
    rng = rng_for(cfg.seed, TAG_ROUTER, layer, attempt)
    return (rng.standard_normal((cfg.E, cfg.H)) * 0.05).astype(np.float32)


def make_bias(cfg: MoEConfig, layer: int) -> Optional[np.ndarray]:
    """Zipf(s=1.1) popularity bias: expert pi(r) gets -1.1*beta*ln(r), r=1..E,
    beta = 0.5 * sigma_z, sigma_z = 0.05*sqrt(H) (the logit standard deviation)."""
    if not cfg.zipf:
        return None
    perm = rng_for(cfg.seed, TAG_PERM, layer).permutation(cfg.E)
    beta = 0.5 * 0.05 * math.sqrt(cfg.H)
    b = np.empty(cfg.E, dtype=np.float64)
    b[perm] = -1.1 * beta * np.log(np.arange(1, cfg.E + 1, dtype=np.float64))
    return b.astype(np.float32)


def _x_draw(rng: np.random.Generator, shape, x_dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape)
    if x_dtype == "bf16":
        return bf16_bits_to_f32(to_bf16_bits(x.astype(np.float32)))
    return x.astype(np.float32)


# --------------------------------------------------------------------------
# workload filter: top-k margin of the router logits
# --------------------------------------------------------------------------
def topk_margins(W: np.ndarray, b: Optional[np.ndarray], x: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit per row of x (fp64).
    Rows of x are tokens.  Returns +inf where k == E."""
    E = W.shape[0]
    if k >= E:
        return np.full(x.shape[0], np.inf)
    z = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T
    if b is not None:
        z = z + np.asarray(b, np.float64)
    part = -np.partition(-z, k, axis=1)[:, : k + 1]
    part.sort(axis=1)
    return part[:, 1] - part[:, 0]       # (k-th largest) - ((k+1)-th largest)


class Workload:
    """All inputs of one configuration, generated lazily and deterministically."""

    def __init__(self, cfg: MoEConfig):
        self.cfg = cfg
        self.layout = record_layout(cfg.H, cfg.I)
        self._routers: Dict[int, np.ndarray] = {}
        self._x: Optional[np.ndarray] = None
        self.redraws = 0

    # -- router ------------------------------------------------------------
    def router(self, layer: int) -> np.ndarray:
        if layer not in self._routers:
            self._routers[layer] = self._make_router(layer)
        return self._routers[layer]

    def bias(self, layer: int) -> Optional[np.ndarray]:
        return make_bias(self.cfg, layer)

    def _make_router(self, layer: int) -> np.ndarray:
        cfg = self.cfg
        if not cfg.redraw_router:
            return make_router(cfg, layer)
        # draw W until every token of this layer meets the margin
        x = self._raw_inputs()
        for attempt in range(1000):
            W = make_router(cfg, layer, attempt)
            xl = x[:, layer, :] if x.ndim == 3 else x
            if np.all(topk_margins(W, self.bias(layer), xl, cfg.k) >= MARGIN):
                return W
        raise RuntimeError("router redraw did not converge")

    # -- inputs --------------------------------------------------------------
    def _raw_inputs(self) -> np.ndarray:
        cfg = self.cfg
        rng = rng_for(cfg.seed, TAG_INPUT)
        if cfg.batched:
            return _x_draw(rng, (cfg.tokens, cfg.H), cfg.x_dtype)
        return _x_draw(rng, (cfg.tokens, cfg.layers, cfg.H), cfg.x_dtype)

    def inputs(self) -> np.ndarray:
        """x [T, L, H] (decode) or [T, H] (batched), fp32 values (bf16-exact
        for bf16 workloads), with margin redraws applied."""
        if self._x is not None:
            return self._x
        cfg = self.cfg
        x = self._raw_inputs()
        if not cfg.redraw_router:
            layers = [0] if cfg.batched else range(cfg.layers)
            for L in layers:
                W, b = self.router(L), self.bias(L)
                xl = x if cfg.batched else x[:, L, :]
                m = topk_margins(W, b, xl, cfg.k)
                for t in np.nonzero(m < MARGIN)[0]:
                    for attempt in range(1000):
                        rng = rng_for(cfg.seed, TAG_REDRAW, int(t), L, attempt)
                        cand = _x_draw(rng, (1, cfg.H), cfg.x_dtype)
                        self.redraws += 1
                        if topk_margins(W, b, cand, cfg.k)[0] >= MARGIN:
                            xl[t] = cand[0]
                            break
                    else:
                        raise RuntimeError("input redraw did not converge")
        self._x = x
        return x

    # -- experts -------------------------------------------------------------
    def record(self, layer: int, expert: int) -> np.ndarray:
        return make_record(self.cfg, layer, expert)

    def shared(self, layer: int) -> Optional[np.ndarray]:
        return make_shared(self.cfg, layer) if self.cfg.shared else None

    def fill_records(self, keys: Sequence[Tuple[int, int]], dests: Sequence[np.ndarray],
                     threads: Optional[int] = None) -> None:
        """Fill many records in parallel (numpy releases the GIL while drawing)."""
        threads = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda kd: fill_record(kd[1], self.cfg, kd[0][0], kd[0][1]),
                        zip(keys, dests)))


def expert_bytes(cfg: MoEConfig) -> int:
    """Unpadded bytes of one routed expert record (codes + scales + codebooks)."""
    return record_layout(cfg.H, cfg.I).nbytes


def expert_bytes_per_token(cfg: MoEConfig) -> int:
    """Expert-weight bytes one token reads over all layers: k routed records
    plus the dense shared expert, per layer."""
    per_layer = cfg.k * expert_bytes(cfg)
    if cfg.shared:
        per_layer += shared_record_bytes(cfg.H, cfg.I)
    return per_layer * cfg.layers
