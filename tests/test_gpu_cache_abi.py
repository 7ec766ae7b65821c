"""The public expert-cache calls of the C ABI driven directly on the GPU:
expert_cache_create, lookup, insert, wait, release, slot_ptr, trace and
destroy (WISP launch post, section "통찰": LRU promotion of the experts the
router keeps choosing; WASTE article, section "유휴 가중치는 메모리가 아니라
제때 닿기만 하면 된다": one copy of one record per miss).

Checked: the trace of a get-or-insert key string against the oracle's LRU
(bit for bit), every slot's bytes against its host record after
expert_cache_wait, the duplicate-insert and bad-slot errors, that an
evicting copy waits for the last reader of its slot (release), and that a
reader after wait sees the new record even when the copy is queued behind
other work."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lru_hand_trace.json")
SLOT = 256 * 1024          # bytes per slot (a multiple of 256)
MOE_E_STATE = -4


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_streaming_amd as m
    m.lib()
    return m


def _host_records(n: int, seed: int) -> torch.Tensor:
    """n pinned host records of SLOT random bytes each (all distinct)."""
    t = torch.empty((n, SLOT), dtype=torch.uint8, pin_memory=True)
    t.numpy()[:] = np.random.default_rng(seed).integers(0, 256, (n, SLOT), dtype=np.uint8)
    return t


def _spin(stream: torch.cuda.Stream, ms: float = 50.0):
    """Keep `stream` busy for a bounded time (a spinning kernel), so that work
    queued behind it lands later than work on other streams."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(ms * 1e-3 * 2.0e9))


def _drive(moe, cache, keys, host, compute, copy):
    """Get-or-insert each key in order; each slot is read on the compute
    stream after expert_cache_wait and released afterwards.  Returns the
    (key, slot, bytes read) of every access."""
    reads = []
    for key in keys:
        s = cache.lookup(int(key))
        if s < 0:
            s, _ = cache.insert(int(key), host[int(key)].data_ptr(), copy)
        assert cache.slot_ptr(s) == cache.pool.data_ptr() + s * SLOT
        cache.wait(s, compute)
        with torch.cuda.stream(compute):
            got = cache.pool[s * SLOT:(s + 1) * SLOT].clone()
        cache.release(s, compute)
        reads.append((int(key), s, got))
    torch.cuda.synchronize()
    return reads


def _check_against_oracle(cache, keys, capacity, reads, host):
    hit, slot, ev = oracle.lru(np.asarray(keys, np.int64), capacity)
    tr = cache.trace()
    assert [r[0] for r in tr] == [int(k) for k in keys]
    assert [r[1] for r in tr] == hit.tolist()
    assert [r[2] for r in tr] == slot.tolist()
    assert [(-1 if r[3] is None else r[3]) for r in tr] == ev.tolist()
    for key, s, got in reads:
        assert torch.equal(got.cpu(), host[key]), f"slot {s} does not hold key {key}'s record"
    return hit


def test_cache_abi_hand_trace(moe):
    g = json.load(open(GOLDEN))
    cap, keys = g["capacity"], g["keys"]
    host = _host_records(max(keys) + 1, 11)
    pool = torch.empty(cap * SLOT, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(cap, SLOT, pool)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    reads = _drive(moe, cache, keys, host, compute, copy)
    hit = _check_against_oracle(cache, keys, cap, reads, host)
    # the fixture's own values, too
    tr = cache.trace()
    assert hit.tolist() == g["hit"]
    assert [r[2] for r in tr] == g["slot"]
    assert [(-1 if r[3] is None else r[3]) for r in tr] == g["evicted"]
    st = cache.stats()
    assert st["lookups"] == len(keys) and st["hits"] == sum(g["hit"])
    assert st["inserts"] == len(keys) - sum(g["hit"]) and st["evictions"] == sum(e >= 0 for e in g["evicted"])
    cache.close()


def test_cache_abi_zipf_string(moe):
    # a longer key string with a skewed popularity (Zipf, s = 1.1) over 96
    # keys through 24 slots: hits, misses and evictions in every order
    rng = np.random.default_rng(5)
    nkeys, cap = 96, 24
    p = 1.0 / np.arange(1, nkeys + 1) ** 1.1
    keys = rng.permutation(nkeys)[rng.choice(nkeys, size=600, p=p / p.sum())]
    host = _host_records(nkeys, 12)
    pool = torch.empty(cap * SLOT, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(cap, SLOT, pool)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    reads = _drive(moe, cache, keys, host, compute, copy)
    hit = _check_against_oracle(cache, keys, cap, reads, host)
    log(f"zipf string: {int(hit.sum())} hits of {len(keys)}, {cache.stats()['evictions']} evictions")
    assert 0 < hit.sum() < len(keys) and cache.stats()["evictions"] > 0
    cache.close()


def test_cache_abi_errors(moe):
    host = _host_records(3, 13)
    pool = torch.empty(2 * SLOT, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(2, SLOT, pool)
    copy = torch.cuda.Stream()
    s, ev = cache.insert(7, host[0].data_ptr(), copy)
    assert (s, ev) == (0, None)
    n_trace = len(cache.trace())
    with pytest.raises(moe.MoeError) as e:
        cache.insert(7, host[1].data_ptr(), copy)          # already cached
    assert e.value.code == MOE_E_STATE
    assert len(cache.trace()) == n_trace and cache.lookup(7) == 0
    with pytest.raises(moe.MoeError) as e:
        cache.wait(1)                                      # never filled
    assert e.value.code == MOE_E_STATE
    for bad in (-1, 2):
        with pytest.raises(moe.MoeError) as e:
            cache.wait(bad)
        assert e.value.code == MOE_E_STATE
        with pytest.raises(moe.MoeError) as e:
            cache.release(bad)
        assert e.value.code == MOE_E_STATE
        with pytest.raises(moe.MoeError) as e:
            cache.slot_ptr(bad)
        assert e.value.code == MOE_E_STATE
    torch.cuda.synchronize()
    cache.close()


def test_cache_abi_eviction_waits_for_last_reader(moe):
    # capacity 1: key A is read on a compute stream kept busy first, then
    # released; key B's insert evicts A into the same slot on the copy
    # stream.  The copy must wait for A's last reader, so the reader sees A.
    # Then the copy stream is kept busy and key C is inserted: a reader
    # after expert_cache_wait must see C, not B.
    host = _host_records(3, 14)
    pool = torch.empty(SLOT, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(1, SLOT, pool)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    s, _ = cache.insert(0, host[0].data_ptr(), copy)
    cache.wait(s, compute)
    _spin(compute)
    with torch.cuda.stream(compute):
        read_a = pool.clone()
    cache.release(s, compute)
    s2, ev = cache.insert(1, host[1].data_ptr(), copy)
    assert (s2, ev) == (s, 0)
    cache.wait(s2, compute)
    with torch.cuda.stream(compute):
        read_b = pool.clone()
    cache.release(s2, compute)
    torch.cuda.synchronize()
    assert torch.equal(read_a.cpu(), host[0]), "the evicting copy overwrote the slot before its reader ran"
    assert torch.equal(read_b.cpu(), host[1])
    _spin(copy)
    s3, ev = cache.insert(2, host[2].data_ptr(), copy)
    assert (s3, ev) == (s, 1)
    cache.wait(s3, compute)
    with torch.cuda.stream(compute):
        read_c = pool.clone()
    torch.cuda.synchronize()
    assert torch.equal(read_c.cpu(), host[2]), "a reader after expert_cache_wait saw the slot before its copy"
    cache.close()
