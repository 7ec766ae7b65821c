"""Pins of the oracle's two-tier exclusive LRU model (oracle.two_tier).

Against what fixes it besides its own code: a trace simulated by hand
(tests/golden/two_tier_hand_trace.json), the single-level LRU for the upper
tier, and the stack property of exclusive LRU tiers: the upper tier holds
the c1 most recently used keys and the lower tier the next c2, so a key at
recency depth d hits the upper tier iff d < c1 and the lower iff
c1 <= d < c1 + c2; the key demoted is the one at depth c1 - 1 and the key
leaving the lower tier the one at depth c1 + c2 - 1 (WISP launch post,
section "통찰": each lookup goes to the fastest tier holding the expert, LRU
promotion).  Checked by brute force over a recency list."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "two_tier_hand_trace.json")


def test_two_tier_hand_trace():
    g = json.load(open(GOLDEN))
    o = oracle.two_tier(np.array(g["keys"]), g["c1"], g["c2"])
    for name in ("hit1", "slot1", "ev1", "hit2", "slot2", "dslot", "dev"):
        assert o[name].tolist() == g[name], name


def _zipf_keys(rng, n, universe, a=1.1):
    w = 1.0 / np.arange(1, universe + 1) ** a
    return rng.choice(universe, size=n, p=w / w.sum())


@pytest.mark.parametrize("c1,c2,universe", [(1, 1, 5), (2, 3, 9), (4, 4, 12), (8, 16, 60), (16, 5, 40)])
def test_two_tier_stack_property(c1, c2, universe):
    rng = np.random.default_rng(1000 + 7 * c1 + c2)
    keys = _zipf_keys(rng, 600, universe)
    o = oracle.two_tier(keys, c1, c2)
    # the upper tier is a single LRU of c1 slots
    h, s, e = oracle.lru(keys, c1)
    assert o["hit1"].tolist() == h.tolist()
    assert o["slot1"].tolist() == s.tolist()
    assert o["ev1"].tolist() == e.tolist()
    # found in either tier exactly where an LRU of c1 + c2 hits
    hb, _, _ = oracle.lru(keys, c1 + c2)
    both = (o["hit1"] == 1) | (o["hit2"] == 1)
    assert both.astype(np.int32).tolist() == hb.tolist()
    # brute force over the recency list (most recent first)
    stack = []
    for i, k in enumerate(keys.tolist()):
        d = stack.index(k) if k in stack else -1
        assert o["hit1"][i] == int(0 <= d < c1)
        if o["hit1"][i]:
            assert o["hit2"][i] == -1 and o["dslot"][i] == -1
        else:
            assert o["hit2"][i] == int(c1 <= d < c1 + c2)
            assert (o["slot2"][i] >= 0) == bool(o["hit2"][i])
            demoted = stack[c1 - 1] if len(stack) >= c1 else -1
            assert o["ev1"][i] == demoted
            # leaves the lower tier: the key at depth c1 + c2 - 1, when the key
            # was in neither tier and both are full
            leaving = stack[c1 + c2 - 1] if (d < 0 or d >= c1 + c2) and len(stack) >= c1 + c2 else -1
            assert o["dev"][i] == leaving
            assert (o["dslot"][i] >= 0) == (demoted != -1)
        if d >= 0:
            stack.pop(d)
        stack.insert(0, k)
    # slots stay in range; a lower slot is never held by two keys
    assert o["slot1"].max() < c1 and o["dslot"].max() < c2 and o["slot2"].max() < c2
