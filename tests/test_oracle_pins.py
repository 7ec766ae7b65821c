"""Pins of the CPU oracle to things other than itself.

Each test checks an oracle function against a library routine, a closed form
with independently constructed inputs, brute force, a published algorithm
(Mattson stack distances) or a hand-worked fixture, chosen so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- values
def test_half_to_double_all_bit_patterns(oracle_lib):
    # every binary16 pattern against numpy's IEEE conversion (library routine)
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_to_double(oracle_lib):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 65536, 4000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]            # finite only
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle_lib.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------- format
@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_layout_matches_synth_and_three_bits(oracle_lib, name):
    cfg = synth.CONFIGS[name]
    off, size, nb, pad = oracle_lib.record_layout(cfg.H, cfg.I)
    lay = synth.record_layout(cfg.H, cfg.I)
    assert tuple(off) == lay.offsets and tuple(size) == lay.sizes
    assert nb == lay.nbytes and pad == lay.padded and pad % 4096 == 0
    # 3.00 bits per weight: two 12-bit indices per group of 8 weights
    weights = 3 * cfg.H * cfg.I
    assert (size[0] + size[1] + size[2]) * 8 == 3 * weights


def test_layout_known_sizes(oracle_lib):
    # per-expert record sizes of the five workloads (unpadded, padded)
    expect = {(256, 512): (346624, 348160), (4096, 14336): (66322432, 66322432),
              (2304, 1024): (2859520, 2863104), (5120, 2048): (12011520, 12013568)}
    for (H, I), (nb, pad) in expect.items():
        _, _, got_nb, got_pad = oracle_lib.record_layout(H, I)
        assert (got_nb, got_pad) == (nb, pad)


def test_layout_rejects_unaligned(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.record_layout(200, 512)


def test_code_tile_bytes_hand_worked(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "code_tile_bytes.json")))
    N, K = g["N"], g["K"]
    v = np.zeros((N, K // 8), np.uint32)
    for c in g["cases"]:
        v[c["r"], c["q"]] = c["v"]
    packed = synth.pack_codes(v)
    for c in g["cases"]:
        assert [int(packed[o]) for o in c["offsets"]] == c["bytes"]
        assert oracle_lib.code_pair(packed, K, c["r"], c["q"]) == c["v"]


def test_code_pair_exhaustive_roundtrip(oracle_lib):
    # all 2^24 code pairs, packed by synth, read back by the oracle's reader
    N, K = 16384, 8192
    v = np.arange(1 << 24, dtype=np.uint32).reshape(N, K // 8)
    packed = synth.pack_codes(v)
    assert np.array_equal(synth.unpack_codes(packed, N, K), v)
    L = oracle_lib.lib()
    import ctypes
    rng = np.random.default_rng(1)
    rows = rng.integers(0, N, 64)
    for r in rows:
        for q in rng.integers(0, K // 8, 64):
            assert L.oracle_code_pair(packed.ctypes.data, K, int(r), int(q)) == v[r, q]


# ---------------------------------------------------------------- decoding
def _onehot_codebook():
    """C[c][i] = (c // 8) if i == c % 8 else 0: integer one-hot rows (exact)."""
    cb = np.zeros((4096, 8), np.float16)
    c = np.arange(4096)
    cb[c, c % 8] = (c // 8).astype(np.float16)
    return cb


def _encode_target(rng, N, K):
    """Random target weights with two (position, value) entries per group and
    the code pairs that produce them under the one-hot codebook."""
    G = K // 8
    i1, i2 = rng.integers(0, 8, (N, G)), rng.integers(0, 8, (N, G))
    v1, v2 = rng.integers(0, 512, (N, G)), rng.integers(0, 512, (N, G))
    target = np.zeros((N, G, 8))
    np.add.at(target, (np.arange(N)[:, None], np.arange(G)[None, :], i1), v1)
    np.add.at(target, (np.arange(N)[:, None], np.arange(G)[None, :], i2), v2)
    a, b = 8 * v1 + i1, 8 * v2 + i2
    codes = (a | (b << 12)).astype(np.uint32)
    return target.reshape(N, K), codes


def test_decode_onehot_target(oracle_lib):
    rng = np.random.default_rng(2)
    N, K = 128, 256
    target, codes = _encode_target(rng, N, K)
    scale = (2.0 ** -rng.integers(3, 8, N)).astype(np.float16)    # exact powers of two
    sec = synth.pack_codes(codes)
    cb = _onehot_codebook()
    for r in range(N):
        w = oracle_lib.decode_row(sec, scale, cb, N, K, r)
        assert np.array_equal(w, float(scale[r]) * target[r])


def test_decode_a_equals_b_doubles(oracle_lib):
    rng = np.random.default_rng(3)
    N, K = 64, 128
    a = rng.integers(0, 4096, (N, K // 8)).astype(np.uint32)
    cb = (rng.standard_normal((4096, 8)) / math.sqrt(2)).astype(np.float16)
    sc = rng.uniform(0.01, 0.03, N).astype(np.float16)
    sec = synth.pack_codes(a | (a << 12))
    for r in range(0, N, 7):
        w = oracle_lib.decode_row(sec, sc, cb, N, K, r)
        ref = 2.0 * float(sc[r]) * cb[a[r]].astype(np.float64).reshape(-1)
        assert np.array_equal(w, ref)


def test_decode_tiny_against_synth_parts(oracle_lib):
    # every weight of a Tiny expert: oracle decode == numpy gather of the
    # parts that synth's own format reader extracts from the same bytes
    cfg = synth.CONFIGS["tiny"]
    rec = synth.make_record(cfg, 0, 3)
    codes, scales, cbs = synth.record_parts(rec, cfg.H, cfg.I)
    off, size, _, _ = oracle_lib.record_layout(cfg.H, cfg.I)
    dims = [(cfg.I, cfg.H), (cfg.I, cfg.H), (cfg.H, cfg.I)]
    for m, (N, K) in enumerate(dims):
        a, b = synth.split_pair(codes[m])
        C = cbs[m].astype(np.float64)
        ref = scales[m].astype(np.float64)[:, None] * (C[a] + C[b]).reshape(N, K)
        sec = rec[off[m]:off[m] + size[m]]
        for r in range(N):
            assert np.array_equal(oracle_lib.decode_row(sec, scales[m], cbs[m], N, K, r), ref[r])


def test_gemv_matches_numpy_matmul(oracle_lib):
    rng = np.random.default_rng(4)
    N, K, T = 128, 384, 3
    target, codes = _encode_target(rng, N, K)
    scale = np.full(N, 0.25, np.float16)
    sec = synth.pack_codes(codes)
    x = rng.standard_normal((T, K))
    y = oracle_lib.rvq_gemv(sec, scale, _onehot_codebook(), N, K, x)
    ref = x @ (0.25 * target).T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-10)
    # unit vector picks out a column
    e = np.zeros((1, K)); e[0, 77] = 1.0
    col = oracle_lib.rvq_gemv(sec, scale, _onehot_codebook(), N, K, e)[0]
    assert np.array_equal(col, 0.25 * target[:, 77])


def test_gemv_threads_do_not_change_results(oracle_lib):
    cfg = synth.CONFIGS["tiny"]
    rec = synth.make_record(cfg, 0, 1)
    off, size, _, _ = oracle_lib.record_layout(cfg.H, cfg.I)
    _, scales, cbs = synth.record_parts(rec, cfg.H, cfg.I)
    x = np.random.default_rng(5).standard_normal((2, cfg.H))
    sec = rec[off[0]:off[0] + size[0]]
    oracle_lib.set_threads(1)
    y1 = oracle_lib.rvq_gemv(sec, scales[0], cbs[0], cfg.I, cfg.H, x)
    oracle_lib.set_threads(5)
    y5 = oracle_lib.rvq_gemv(sec, scales[0], cbs[0], cfg.I, cfg.H, x)
    oracle_lib.set_threads(1)
    assert np.array_equal(y1, y5)


# ------------------------------------------------------------- expert FFN
def _dense_swiglu(Wg, Wu, Wd, x):
    """Textbook SwiGLU in torch fp64: down(silu(gate x) * (up x))."""
    x = torch.as_tensor(x, dtype=torch.float64)
    g = x @ torch.as_tensor(Wg).T
    u = x @ torch.as_tensor(Wu).T
    return ((torch.nn.functional.silu(g) * u) @ torch.as_tensor(Wd).T).numpy()


def test_expert_ffn_equals_dense_swiglu_onehot(oracle_lib):
    rng = np.random.default_rng(6)
    H, I = 128, 256
    tg, cg = _encode_target(rng, I, H)
    tu, cu = _encode_target(rng, I, H)
    td, cd = _encode_target(rng, H, I)
    s = 2.0 ** -9
    scales = (np.full(I, s, np.float16), np.full(I, s, np.float16), np.full(H, s, np.float16))
    cb = _onehot_codebook()
    rec = synth.build_record(H, I, cg, cu, cd, scales, np.stack([cb, cb, cb]))
    x = rng.standard_normal((3, H))
    y = oracle_lib.expert_ffn(rec, H, I, x)
    ref = _dense_swiglu(s * tg, s * tu, s * td, x)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_expert_ffn_equals_dense_swiglu_random(oracle_lib):
    # random Tiny record, weights materialised from synth's parts
    cfg = synth.CONFIGS["tiny"]
    rec = synth.make_record(cfg, 0, 5)
    codes, scales, cbs = synth.record_parts(rec, cfg.H, cfg.I)
    Ws = []
    for m in range(3):
        a, b = synth.split_pair(codes[m])
        C = cbs[m].astype(np.float64)
        Ws.append(scales[m].astype(np.float64)[:, None] * (C[a] + C[b]).reshape(codes[m].shape[0], -1))
    x = np.random.default_rng(7).standard_normal((4, cfg.H))
    np.testing.assert_allclose(oracle_lib.expert_ffn(rec, cfg.H, cfg.I, x),
                               _dense_swiglu(*Ws, x), rtol=1e-11, atol=1e-13)


def test_expert_ffn_zero_codebook_gives_zero(oracle_lib):
    cfg = synth.CONFIGS["tiny"]
    rec = synth.make_record(cfg, 0, 0).copy()
    off, size, _, _ = oracle_lib.record_layout(cfg.H, cfg.I)
    for m in (6, 7, 8):
        rec[off[m]:off[m] + size[m]] = 0
    y = oracle_lib.expert_ffn(rec, cfg.H, cfg.I, np.ones((1, cfg.H)))
    assert np.all(y == 0.0)


def test_shared_ffn_equals_dense_swiglu(oracle_lib):
    rng = np.random.default_rng(8)
    H, I = 128, 256
    bits = synth.to_bf16_bits(rng.standard_normal(3 * H * I).astype(np.float32) * 0.02)
    w = synth.bf16_bits_to_f32(bits).astype(np.float64)
    Wg, Wu, Wd = w[:I * H].reshape(I, H), w[I * H:2 * I * H].reshape(I, H), w[2 * I * H:].reshape(H, I)
    x = rng.standard_normal((2, H))
    np.testing.assert_allclose(oracle_lib.shared_ffn(bits, H, I, x), _dense_swiglu(Wg, Wu, Wd, x),
                               rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- routing
def test_route_logits_match_matmul(oracle_lib):
    rng = np.random.default_rng(9)
    E, H = 16, 96
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    x = rng.standard_normal((5, H))
    _, _, z = oracle_lib.route(W, b, x, 3, "softmax")
    np.testing.assert_allclose(z, x @ W.astype(np.float64).T + b.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_route_tiny_bruteforce_subsets(oracle_lib):
    cfg = synth.CONFIGS["tiny"]
    wl = synth.Workload(cfg)
    W, x = wl.router(0), wl.inputs()[:, 0, :].astype(np.float64)
    idx, w, z = oracle_lib.route(W, None, x, cfg.k, cfg.score)
    for t in range(cfg.tokens):
        # the selected set is the unique k-subset with the largest logit sum
        sums = {S: z[t, list(S)].sum() for S in itertools.combinations(range(cfg.E), cfg.k)}
        best = max(sums, key=sums.get)
        assert sorted(best) == sorted(idx[t].tolist())
        second = sorted(sums.values())[-2]
        assert sums[best] - second >= synth.MARGIN * 0.999
        # softmax over all experts, renormalised over S (scipy routine)
        p = scipy.special.softmax(z[t])
        np.testing.assert_allclose(w[t], p[idx[t]] / p[idx[t]].sum(), rtol=1e-12)
        assert abs(w[t].sum() - 1.0) <= 1e-12


def test_route_sigmoid_renorm(oracle_lib):
    rng = np.random.default_rng(10)
    E, H, k = 64, 128, 8
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32)
    x = rng.standard_normal((6, H))
    idx, w, z = oracle_lib.route(W, b, x, k, "sigmoid")
    for t in range(6):
        order = np.lexsort((np.arange(E), -z[t]))      # z desc, id asc
        assert idx[t].tolist() == order[:k].tolist()
        s = scipy.special.expit(z[t, idx[t]])
        np.testing.assert_allclose(w[t], s / s.sum(), rtol=1e-12)
        assert abs(w[t].sum() - 1.0) <= 1e-12


def test_route_k_equals_E_is_full_softmax(oracle_lib):
    rng = np.random.default_rng(11)
    E, H = 8, 64
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    x = rng.standard_normal((3, H))
    idx, w, z = oracle_lib.route(W, None, x, E, "softmax")
    for t in range(3):
        full = scipy.special.softmax(z[t])
        np.testing.assert_allclose(w[t], full[idx[t]], rtol=1e-12)


def test_route_k1_weight_one(oracle_lib):
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    x = rng.standard_normal((4, 64))
    for score in ("softmax", "sigmoid"):
        idx, w, z = oracle_lib.route(W, None, x, 1, score)
        assert np.all(w == 1.0)
        assert np.array_equal(idx[:, 0], np.argmax(z, axis=1))


def test_route_ties_prefer_lower_id(oracle_lib):
    W = np.zeros((6, 4), np.float32)
    W[1] = W[4] = [1, 0, 0, 0]        # experts 1 and 4 tie on the top logit
    W[2] = [0.5, 0, 0, 0]
    x = np.array([[1.0, 0, 0, 0]])
    idx, w, _ = oracle_lib.route(W, None, x, 2, "softmax")
    assert idx[0].tolist() == [1, 4]
    idx, _, _ = oracle_lib.route(W, None, x, 3, "sigmoid")
    assert idx[0].tolist() == [1, 4, 2]


# ------------------------------------------------------------------ layer
def test_layer_identical_experts_equals_single_expert(oracle_lib):
    cfg = synth.CONFIGS["tiny"]
    rec = synth.make_record(cfg, 0, 2)
    wl = synth.Workload(cfg)
    x = wl.inputs()[:, 0, :].astype(np.float64)
    out, idx, w = oracle_lib.layer(wl.router(0), None, cfg.k, cfg.score, [rec] * cfg.E, None,
                                   cfg.H, cfg.I, x)
    np.testing.assert_allclose(out, oracle_lib.expert_ffn(rec, cfg.H, cfg.I, x), rtol=1e-12, atol=1e-14)


def test_layer_shared_term_is_additive(oracle_lib):
    rng = np.random.default_rng(13)
    cfg = synth.CONFIGS["tiny"].replace(shared=True, E=4, score="sigmoid")
    recs = [synth.make_record(cfg, 0, e) for e in range(cfg.E)]
    sh = synth.make_shared(cfg, 0)
    W = (rng.standard_normal((cfg.E, cfg.H)) * 0.05).astype(np.float32)
    x = rng.standard_normal((2, cfg.H))
    with_sh, _, _ = oracle_lib.layer(W, None, 2, "sigmoid", recs, sh, cfg.H, cfg.I, x)
    no_sh, _, _ = oracle_lib.layer(W, None, 2, "sigmoid", recs, None, cfg.H, cfg.I, x)
    np.testing.assert_allclose(with_sh - no_sh, oracle_lib.shared_ffn(sh, cfg.H, cfg.I, x),
                               rtol=1e-10, atol=1e-14)


def test_layer_one_expert_identity_router_is_dense_ffn(oracle_lib):
    # E = 1, k = 1: routing is the identity and the layer is one dense SwiGLU
    rng = np.random.default_rng(14)
    H, I = 128, 128
    tg, cg = _encode_target(rng, I, H)
    tu, cu = _encode_target(rng, I, H)
    td, cd = _encode_target(rng, H, I)
    s = 2.0 ** -9
    cb = _onehot_codebook()
    sc = (np.full(I, s, np.float16), np.full(I, s, np.float16), np.full(H, s, np.float16))
    rec = synth.build_record(H, I, cg, cu, cd, sc, np.stack([cb, cb, cb]))
    W = rng.standard_normal((1, H)).astype(np.float32)
    x = rng.standard_normal((3, H))
    out, idx, w = oracle_lib.layer(W, None, 1, "softmax", [rec], None, H, I, x)
    assert np.all(idx == 0) and np.all(w == 1.0)
    np.testing.assert_allclose(out, _dense_swiglu(s * tg, s * tu, s * td, x), rtol=1e-12, atol=1e-12)


def test_layer_combine_weights(oracle_lib):
    cfg = synth.CONFIGS["tiny"]
    wl = synth.Workload(cfg)
    recs = [wl.record(0, e) for e in range(cfg.E)]
    x = wl.inputs()[:, 0, :].astype(np.float64)
    out, idx, w = oracle_lib.layer(wl.router(0), None, cfg.k, cfg.score, recs, None, cfg.H, cfg.I, x)
    for t in range(cfg.tokens):
        ref = sum(w[t, j] * oracle_lib.expert_ffn(recs[idx[t, j]], cfg.H, cfg.I, x[t:t + 1])[0]
                  for j in range(cfg.k))
        np.testing.assert_allclose(out[t], ref, rtol=1e-13, atol=1e-15)


# -------------------------------------------------------------------- LRU
def test_lru_hand_trace(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "lru_hand_trace.json")))
    hit, slot, ev = oracle_lib.lru(g["keys"], g["capacity"])
    assert hit.tolist() == g["hit"]
    assert slot.tolist() == g["slot"]
    assert ev.tolist() == g["evicted"]


def _stack_distance_hits(keys, capacity):
    """Mattson et al. (1970): an LRU access hits iff the number of distinct
    keys referenced since the previous access to the same key is < capacity."""
    hits, last = [], {}
    for i, k in enumerate(keys):
        if k in last:
            hits.append(int(len(set(keys[last[k] + 1:i])) < capacity))
        else:
            hits.append(0)
        last[k] = i
    return hits


@pytest.mark.parametrize("capacity", [1, 2, 5, 17, 64])
def test_lru_matches_stack_distance(oracle_lib, capacity):
    rng = np.random.default_rng(capacity)
    p = 1.0 / np.arange(1, 101) ** 1.1
    keys = rng.choice(100, 1500, p=p / p.sum()).tolist()
    hit, slot, ev = oracle_lib.lru(keys, capacity)
    assert hit.tolist() == _stack_distance_hits(keys, capacity)


def test_lru_inclusion_and_slot_validity(oracle_lib):
    rng = np.random.default_rng(15)
    keys = rng.integers(0, 40, 800).tolist()
    prev = None
    for cap in range(1, 41):
        hit, slot, ev = oracle_lib.lru(keys, cap)
        if prev is not None:
            assert np.all(hit >= prev)              # hits(C) subset of hits(C+1)
        prev = hit
        # replay: slots hold one key each; hits find the key where it was put
        where, holder = {}, {}
        for i, k in enumerate(keys):
            s = int(slot[i])
            assert 0 <= s < cap
            if hit[i]:
                assert where[k] == s and ev[i] == -1
            else:
                assert k not in where
                if ev[i] >= 0:
                    assert holder[s] == ev[i]
                    del where[int(ev[i])]
                else:
                    assert s not in holder
                where[k], holder[s] = s, k


def test_lru_capacity_extremes(oracle_lib):
    keys = [3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5]
    hit, _, _ = oracle_lib.lru(keys, 100)
    assert int((hit == 0).sum()) == len(set(keys))
    cyc = list(range(6)) * 5          # capacity + 1 keys cycled: every access misses
    hit, _, _ = oracle_lib.lru(cyc, 5)
    assert hit.sum() == 0


def test_stream_trace_ascending_order_and_keys(oracle_lib):
    idx = np.array([[5, 2], [1, 2], [2, 5], [7, 0]], np.int32)   # steps (t, L) with 2 layers
    key, hit, slot, ev = oracle_lib.stream_trace(idx, nlayers=2, E=8, capacity=3)
    # step 0: layer 0, experts 2,5; step 1: layer 1: 1,2; step 2: layer 0: 2,5; step 3: layer 1: 0,7
    assert key.tolist() == [2, 5, 9, 10, 2, 5, 8, 15]
    # by hand, capacity 3: 2,5,9 fill slots 0,1,2; 10 evicts 2 (slot 0); 2 evicts 5
    # (slot 1); 5 evicts 9 (slot 2); 8 evicts 10 (slot 0); 15 evicts 2 (slot 1)
    assert hit.tolist() == [0] * 8
    assert slot.tolist() == [0, 1, 2, 0, 1, 2, 0, 1]
    assert ev.tolist() == [-1, -1, -1, 2, 5, 9, 10, 2]
