"""Hit rate against cache size in one pass: the library's LRU stack distances
(moe_lru_stack_distances, host-only) against the definition by brute force
and against the oracle's linked-list LRU run at each capacity separately.
No GPU: these calls launch no kernel."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def moe():
    import os

    from routed_expert_streaming_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from routed_expert_streaming_amd import build
        build.build()
    import routed_expert_streaming_amd as m
    return m


def brute_distances(keys):
    """Definition: distinct keys strictly between two references to a key."""
    out = []
    for i, k in enumerate(keys):
        prev = [p for p in range(i) if keys[p] == k]
        out.append(-1 if not prev else len(set(keys[prev[-1] + 1:i])))
    return out


def decode_keys(rng, steps, layers, E, k, zipf):
    """Key string of a streamed decode: per (token, layer) the k distinct
    experts it selects, looked up in ascending id, key = layer * E + expert."""
    p = 1.0 / np.arange(1, E + 1) ** zipf
    p /= p.sum()
    perm = [rng.permutation(E) for _ in range(layers)]
    keys = []
    for _ in range(steps):
        for L in range(layers):
            sel = np.sort(perm[L][rng.choice(E, size=k, replace=False, p=p)])
            keys.extend(int(L * E + e) for e in sel)
    return np.array(keys, dtype=np.uint32)


@pytest.mark.parametrize("seed", range(6))
def test_matches_definition(moe, seed):
    rng = np.random.default_rng(seed)
    keys = rng.integers(0, 1 + 3 * seed, size=60).tolist()
    assert moe.lru_stack_distances(keys).tolist() == brute_distances(keys)


def test_worked_example(moe):
    # a b a c b a a: a at 2 after {b}; b at 4 after {a, c}; a at 5 after {c, b}
    d = moe.lru_stack_distances([1, 2, 1, 3, 2, 1, 1])
    assert d.tolist() == [-1, -1, 1, -1, 2, 2, 0]
    assert moe.lru_hits_at(d, [1, 2, 3, 4]) == [1, 2, 4, 4]


def test_edge_cases(moe):
    assert moe.lru_stack_distances([]).size == 0
    assert moe.lru_stack_distances([7] * 5).tolist() == [-1, 0, 0, 0, 0]
    assert moe.lru_stack_distances(np.arange(100)).tolist() == [-1] * 100
    assert moe.lru_stack_distances([0xFFFFFFFF, 0, 0xFFFFFFFF]).tolist() == [-1, -1, 1]
    assert moe.lru_hits_at(np.array([], np.int32), [1, 10]) == [0, 0]


def test_rejects_bad_arguments(moe):
    from routed_expert_streaming_amd._lib import MOE_E_INVAL
    L = moe.lib()
    assert L.moe_lru_stack_distances(None, -1, None) == MOE_E_INVAL
    assert L.moe_lru_stack_distances(None, 3, None) == MOE_E_INVAL
    assert L.moe_lru_stack_distances(None, 0, None) == 0


@pytest.mark.parametrize("zipf", [0.0, 0.9])
def test_every_capacity_equals_a_separate_lru_run(moe, zipf):
    # decode-shaped key string (8 layers x 96 experts, top-6): the one-pass
    # curve must equal the oracle's LRU, reference by reference, at every
    # capacity tried, from below k to above the number of keys
    rng = np.random.default_rng(11)
    keys = decode_keys(rng, steps=120, layers=8, E=96, k=6, zipf=zipf)
    d = moe.lru_stack_distances(keys)
    caps = [1, 5, 6, 7, 48, 96, 192, 384, 500, 768, 769, 5000]
    pred = moe.lru_hits_at(d, caps)
    for c, hits in zip(caps, pred):
        hit, _, _ = oracle.lru(keys.astype(np.int64), c)
        assert np.array_equal(hit.astype(bool), (d >= 0) & (d < c)), c
        assert int(hit.sum()) == hits, c
    # more capacity never loses a hit (LRU is a stack algorithm), and a cache
    # holding every key misses only first references
    assert all(a <= b for a, b in zip(pred, pred[1:]))
    assert pred[-1] == keys.size - len(np.unique(keys))
