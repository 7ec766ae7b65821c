"""The K3-scale streaming slice at its own size: 8 layers x 768 experts
(6144 records of 12 MB in host memory, page-locked up to 52 GiB and the rest
pageable), a cold HBM slot cache of 25% of the records (1536 slots), top-16
sigmoid routing with the Zipf popularity bias, one token at a time.

The cache trace of the whole decode (every lookup: key, hit, slot, evicted
key) must equal, bit for bit, the oracle's LRU run over the oracle's own
routing (WISP launch post, section "통찰": LRU promotion; WARP article,
section "WARP의 캐시 설정에서 드러나는 역설": hit rate against cache size).
Layer outputs at sampled steps are checked against the oracle's layer."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import RTOL_F32_PATH, log, rel_l2, same_sets

pytestmark = pytest.mark.gpu

TOKENS = 64


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_streaming_amd as m
    m.lib()
    return m


def test_k3_slice_full_scale_trace(moe):
    from routed_expert_streaming_amd.device_workload import DeviceWorkload, HostRecordPool
    cfg = synth.get_config("k3_slice", tokens=TOKENS)
    assert (cfg.layers, cfg.E, cfg.k, cfg.cache_capacity) == (8, 768, 16, 1536)
    log(f"k3 slice: {cfg.layers * cfg.E} records into host memory")
    dw = DeviceWorkload(cfg, with_records=False)
    hp = HostRecordPool(cfg, list(range(cfg.layers)))
    log(f"  {hp.pinned_records} of {cfg.layers * cfg.E} records page-locked")
    tables = [hp.table(L) for L in range(cfg.layers)]
    cap = cfg.cache_capacity
    pool = torch.empty(cap * hp.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(cap, hp.stride, pool)
    x = dw.inputs()
    copy_stream = torch.cuda.Stream()
    ws = torch.empty(moe.streamed_workspace_bytes(dw.layers[0]), dtype=torch.uint8, device="cuda")
    out = torch.empty((TOKENS, cfg.layers, cfg.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((TOKENS, cfg.layers, cfg.k), dtype=torch.int32, device="cuda")
    for t in range(TOKENS):
        for L in range(cfg.layers):
            moe.layer_forward_streamed(dw.layers[L], cache, L, None, x[t, L][None], copy_stream, ws=ws,
                                       out=out[t, L][None], idx=idx[t, L][None], host_table=tables[L])
    torch.cuda.synchronize()
    tr = cache.trace()
    st = cache.stats()
    log(f"  {TOKENS} tokens: hits {st['hits']}/{st['lookups']}, evictions {st['evictions']}")
    assert st["evictions"] > 0, "the decode should fill the cache and evict"

    # the oracle's routing for every (token, layer), then its LRU over those keys
    x64 = x.cpu().numpy().astype(np.float64)
    oidx = np.zeros((TOKENS * cfg.layers, cfg.k), np.int32)
    for L in range(cfg.layers):
        ridx, _, _ = oracle.route(dw.wl.router(L), dw.wl.bias(L), x64[:, L, :], cfg.k, cfg.score)
        oidx[L::cfg.layers] = ridx
    gidx = idx.cpu().numpy().reshape(TOKENS * cfg.layers, cfg.k)
    assert same_sets(gidx, oidx), "routing differs from the oracle's"
    key, hit, slot, ev = oracle.stream_trace(oidx, cfg.layers, cfg.E, cap)
    assert len(tr) == TOKENS * cfg.layers * cfg.k
    assert [r[0] for r in tr] == key.tolist()
    assert [r[1] for r in tr] == hit.tolist()
    assert [r[2] for r in tr] == slot.tolist()
    assert [(-1 if r[3] is None else r[3]) for r in tr] == ev.tolist()
    half = (TOKENS // 2) * cfg.layers * cfg.k
    log(f"  trace equals the oracle's: hit rate {hit.mean():.4f} (tokens {TOKENS // 2}.. {hit[half:].mean():.4f})")

    # layer outputs at sampled steps (cold start, middle, end)
    oracle.set_threads(16)
    empty = np.zeros(1, np.uint8)
    worst = 0.0
    for t, L in [(0, 0), (0, 7), (17, 3), (40, 5), (TOKENS - 1, 0), (TOKENS - 1, 7)]:
        need = set(int(e) for e in oidx[t * cfg.layers + L])
        recs = [dw.wl.record(L, e) if e in need else empty for e in range(cfg.E)]
        ref, _, _ = oracle.layer(dw.wl.router(L), dw.wl.bias(L), cfg.k, cfg.score, recs, dw.wl.shared(L), cfg.H,
                                 cfg.I, x64[t, L][None])
        r = rel_l2(out[t, L].cpu().numpy(), ref[0])
        worst = max(worst, r)
        assert r <= RTOL_F32_PATH, f"token {t} layer {L}: rel_l2 {r:.3e}"
    log(f"  sampled outputs: worst rel_l2 {worst:.3e}")
    cache.close()
    del pool, hp
    torch.cuda.empty_cache()
