"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Expert indices and cache traces are compared bit for bit; outputs by
relative L2 per layer call (<= 1e-3).  Inputs are the seeded synthetic
workloads shared by both sides.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import RTOL_F32_PATH, log, rel_l2, same_sets, weights_by_expert

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_streaming_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def tiny(moe):
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    return DeviceWorkload(synth.CONFIGS["tiny"])


def _oracle_layer(dw, L, x64):
    """Oracle layer output.  Only the experts the oracle's own router selects
    are read, so the others get a placeholder instead of a generated record."""
    cfg, wl = dw.cfg, dw.wl
    ridx, _, _ = oracle.route(wl.router(L), wl.bias(L), x64, cfg.k, cfg.score)
    needed = set(int(e) for e in ridx.reshape(-1))
    empty = np.zeros(1, np.uint8)
    recs = [wl.record(L, e) if e in needed else empty for e in range(cfg.E)]
    return oracle.layer(wl.router(L), wl.bias(L), cfg.k, cfg.score, recs, wl.shared(L), cfg.H, cfg.I, x64)


def test_tiny_route_bit_exact(moe, tiny):
    cfg = tiny.cfg
    x = tiny.inputs()[:, 0, :].contiguous()
    idx, w = moe.route_topk(tiny.layers[0].router, x)
    ridx, rw, z = oracle.route(tiny.wl.router(0), None, x.cpu().numpy().astype(np.float64), cfg.k, cfg.score)
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(idx, ridx)      # margins >= 1e-3 everywhere: order is unique too
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-6)


def test_tiny_layer_parity(moe, tiny):
    x = tiny.inputs()[:, 0, :].contiguous()
    out, idx, w = moe.layer_forward(tiny.layers[0], x)
    ref, ridx, rw = _oracle_layer(tiny, 0, x.cpu().numpy().astype(np.float64))
    assert same_sets(idx.cpu().numpy(), ridx)
    r = rel_l2(out.cpu().numpy(), ref)
    log(f"tiny layer rel_l2={r:.3e}")
    assert r <= RTOL_F32_PATH


def test_tiny_zero_tokens_is_noop(moe, tiny):
    x = torch.empty((0, tiny.cfg.H), device="cuda")
    out, idx, w = moe.layer_forward(tiny.layers[0], x)
    assert out.shape == (0, tiny.cfg.H)


@pytest.mark.parametrize("T", [1, 5])
def test_expert_ffn_parity(moe, tiny, T):
    cfg = tiny.cfg
    rec_np = tiny.wl.record(0, 6)
    rec = torch.from_numpy(rec_np).cuda()
    rng = np.random.default_rng(T)
    x = rng.standard_normal((T, cfg.H)).astype(np.float32)
    g = rng.uniform(0.1, 1.0, T).astype(np.float32)
    y0 = rng.standard_normal((T, cfg.H)).astype(np.float32)
    y = torch.from_numpy(y0).cuda()
    moe.expert_ffn_rvq(rec, cfg.H, cfg.I, torch.from_numpy(x).cuda(), gate_w=torch.from_numpy(g).cuda(), y=y,
                       accumulate=True)
    ffn = oracle.expert_ffn(rec_np, cfg.H, cfg.I, x.astype(np.float64))
    ref = y0 + g[:, None] * ffn
    r = rel_l2(y.cpu().numpy() - y0, g[:, None] * ffn)
    log(f"expert ffn T={T} rel_l2={r:.3e}")
    assert r <= RTOL_F32_PATH
    np.testing.assert_allclose(y.cpu().numpy(), ref, rtol=1e-3, atol=1e-3)


def test_expert_ffn_onehot_exact_codebook(moe):
    # integer one-hot codebook, power-of-two scales, fp16-exact inputs: every
    # product is exact and the sums are small integers, so fp32 equals fp64
    H, I = 256, 256
    rng = np.random.default_rng(3)
    cb = np.zeros((4096, 8), np.float16)
    c = np.arange(4096)
    cb[c, c % 8] = ((c // 8) % 8).astype(np.float16)
    codes = [rng.integers(0, 1 << 24, (n, kk // 8)).astype(np.uint32) for n, kk in ((I, H), (I, H), (H, I))]
    sc = (np.full(I, 2.0 ** -6, np.float16), np.full(I, 2.0 ** -6, np.float16), np.full(H, 2.0 ** -6, np.float16))
    rec_np = synth.build_record(H, I, *codes, sc, np.stack([cb, cb, cb]))
    x = rng.integers(-2, 3, (2, H)).astype(np.float32)
    y = moe.expert_ffn_rvq(torch.from_numpy(rec_np).cuda(), H, I, torch.from_numpy(x).cuda())
    ref = oracle.expert_ffn(rec_np, H, I, x.astype(np.float64))
    assert rel_l2(y.cpu().numpy(), ref) <= RTOL_F32_PATH


@pytest.mark.parametrize("name,T", [("kimi_linear", 6), ("mixtral", 2), ("k3_slice", 2), ("batched", 3)])
def test_layer_parity_real_shapes(moe, name, T):
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    cfg = synth.get_config(name, tokens=T, layers=1, batched=False)
    log(f"layer parity {name} T={T}: uploading")
    dw = DeviceWorkload(cfg, layers=[0])
    x = dw.inputs()
    x = (x[:, 0, :] if x.dim() == 3 else x).contiguous()
    if cfg.x_dtype == "bf16":
        x = x.to(torch.bfloat16)
    oracle.set_threads(16)
    out, idx, w = moe.layer_forward(dw.layers[0], x)
    ref, ridx, rw = _oracle_layer(dw, 0, x.float().cpu().numpy().astype(np.float64))
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    assert same_sets(idx, ridx)
    np.testing.assert_allclose(weights_by_expert(idx, w), weights_by_expert(ridx, rw), rtol=1e-5, atol=1e-7)
    for t in range(T):
        r = rel_l2(out[t].cpu().numpy(), ref[t])
        log(f"  {name} token {t} rel_l2={r:.3e}")
        assert r <= RTOL_F32_PATH
    del dw
    torch.cuda.empty_cache()


def _check_decode(moe, cfg, layers=None, sample=None, method=None, down=None):
    """Persistent decode kernel (one launch for all tokens x layers) against
    the oracle, layer call by layer call; also run-to-run determinism, the
    device-side wait flag and (if given) the gate/up and down methods in use."""
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    log(f"decode {cfg.name}: {cfg.tokens} tokens x {cfg.layers} layers, uploading")
    dw = DeviceWorkload(cfg)
    if method is not None:
        assert moe.decode_gate_up_method(dw.layers) == method
    if down is not None:
        assert moe.decode_down_method(dw.layers) == down
    x = dw.inputs()
    ws = torch.empty(moe.decode_workspace_bytes(dw.layers), dtype=torch.uint8, device="cuda")
    out, idx = moe.decode_forward(dw.layers, x, ws=ws)
    out2, idx2 = moe.decode_forward(dw.layers, x, ws=ws)
    torch.cuda.synchronize()
    assert not moe.decode_status(ws), "device-side wait limit reached"
    assert torch.equal(out, out2) and torch.equal(idx, idx2)
    oracle.set_threads(16)
    x64 = x.cpu().numpy().astype(np.float64)
    steps = [(t, L) for t in range(cfg.tokens) for L in range(cfg.layers)]
    if sample is not None:
        steps = [steps[i] for i in sample]
    worst = 0.0
    for t, L in steps:
        ref, ridx, _ = _oracle_layer(dw, L, x64[t, L][None])
        assert same_sets(idx[t, L].cpu().numpy()[None], ridx), f"routing differs at token {t} layer {L}"
        r = rel_l2(out[t, L].cpu().numpy(), ref[0])
        worst = max(worst, r)
        assert r <= RTOL_F32_PATH, f"token {t} layer {L}: rel_l2 {r:.3e}"
    log(f"  {len(steps)} layer calls checked, worst rel_l2 {worst:.3e}")


def test_decode_forward_two_layers(moe):
    _check_decode(moe, synth.get_config("kimi_linear", tokens=3, layers=2))


def test_decode_forward_tiny(moe):
    # 32 (rank, tile, chunk) units over 256 workgroups: most stay idle
    _check_decode(moe, synth.get_config("tiny", tokens=4))


def test_decode_forward_k3_shape_shared(moe):
    _check_decode(moe, synth.get_config("k3_slice", tokens=2, layers=2), method="gathers")


def test_decode_forward_more_layers_than_one_launch(moe):
    # 45 layers: more than one launch carries (40), so the decode runs one
    # launch per (token, layer group); every layer call against the oracle
    _check_decode(moe, synth.get_config("tiny", tokens=2, layers=45))


def test_decode_forward_no_tokens(moe):
    # T = 0: nothing to decode, no launch, no error
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    dw = DeviceWorkload(synth.get_config("tiny", tokens=1))
    x = torch.empty((0, 1, dw.cfg.H), dtype=torch.float32, device="cuda")
    out, idx = moe.decode_forward(dw.layers, x)
    assert out.shape[0] == 0 and idx.shape[0] == 0


@pytest.mark.parametrize("k", [4, 8])
def test_decode_forward_k3_shape_fewer_experts_per_token(moe, k):
    # num_experts_per_token below the K3 default of 16 (the k sweep's settings)
    _check_decode(moe, synth.get_config("k3_slice", tokens=2, layers=2, k=k))


def _check_decode_all(moe, cfg, method=None, down=None):
    """The whole decode of a configuration (every token x every layer, one
    launch) against the oracle, every layer call; each layer's records are
    generated once, for the experts some token selects."""
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    log(f"decode {cfg.name}: all {cfg.tokens} tokens x {cfg.layers} layers, uploading")
    dw = DeviceWorkload(cfg)
    if method is not None:
        assert moe.decode_gate_up_method(dw.layers) == method
    if down is not None:
        assert moe.decode_down_method(dw.layers) == down
    x = dw.inputs()
    ws = torch.empty(moe.decode_workspace_bytes(dw.layers), dtype=torch.uint8, device="cuda")
    out, idx = moe.decode_forward(dw.layers, x, ws=ws)
    torch.cuda.synchronize()
    assert not moe.decode_status(ws), "device-side wait limit reached"
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    oracle.set_threads(16)
    x64 = x.cpu().numpy().astype(np.float64)
    empty = np.zeros(1, np.uint8)
    rs = []
    for L in range(cfg.layers):
        W, b = dw.wl.router(L), dw.wl.bias(L)
        ridx, _, _ = oracle.route(W, b, x64[:, L], cfg.k, cfg.score)
        assert same_sets(idx[:, L], ridx), f"routing differs at layer {L}"
        need = set(int(e) for e in ridx.reshape(-1))
        recs = [dw.wl.record(L, e) if e in need else empty for e in range(cfg.E)]
        ref, _, _ = oracle.layer(W, b, cfg.k, cfg.score, recs, dw.wl.shared(L), cfg.H, cfg.I, x64[:, L])
        for t in range(cfg.tokens):
            r = rel_l2(out[t, L], ref[t])
            rs.append(r)
            assert r <= RTOL_F32_PATH, f"token {t} layer {L}: rel_l2 {r:.3e}"
        if L % 4 == 3:
            log(f"  layers 0..{L} checked, worst rel_l2 so far {max(rs):.3e}")
    log(f"  {len(rs)} layer calls checked: worst rel_l2 {max(rs):.3e}, median {np.median(rs):.3e}")


def test_decode_forward_mixtral_all_tokens(moe):
    # the configuration bench.py times, whole: all 64 tokens x 32 layers of 8
    # resident experts (gate/up and down by table lookup, the default at
    # I = 14336) in one launch; all 2048 layer calls against the oracle
    _check_decode_all(moe, synth.CONFIGS["mixtral"], method="lookup", down="lookup")


def test_decode_forward_kimi_linear_all_tokens(moe):
    # the Kimi-Linear-class decode, whole: 128 tokens x 27 layers of 256
    # experts + the shared expert, sigmoid top-8 with the Zipf bias (codebook
    # gathers at I = 1024); all 3456 layer calls against the oracle
    _check_decode_all(moe, synth.CONFIGS["kimi_linear"], method="gathers", down="gathers")


def test_decode_forward_mixtral_gathers(moe, monkeypatch):
    # the same shape with gate/up and down by codebook gathers
    monkeypatch.setenv("MOE_DECODE_LUT", "0")
    _check_decode(moe, synth.get_config("mixtral", tokens=1, layers=4), method="gathers", down="gathers")


def test_decode_forward_mixtral_lookup_gate_up_only(moe, monkeypatch):
    # gate/up by table lookup, down by codebook gathers
    monkeypatch.setenv("MOE_DECODE_LUT", "2")
    _check_decode(moe, synth.get_config("mixtral", tokens=1, layers=4), method="lookup", down="gathers")


def test_decode_forward_lut_default_small(moe):
    # table lookup chosen by the shape (I = 8192), not forced: 16 tiles per
    # workgroup, 8 workgroups per segment, several tokens and layers
    _check_decode(moe, synth.get_config("mixtral", H=1024, I=8192, E=4, tokens=3, layers=3), method="lookup",
                  down="lookup")


def test_decode_forward_lut_straddling_segments(moe, monkeypatch):
    # gate/up by table lookup forced at a shape whose default is gathers:
    # 4.5 tiles per workgroup, so ranges straddle segments (matrices, chunk
    # groups, experts) and most waves have no tile
    monkeypatch.setenv("MOE_DECODE_LUT", "1")
    _check_decode(moe, synth.get_config("mixtral", H=2048, I=3072, k=3, tokens=2, layers=2), method="lookup",
                  down="lookup")


def test_decode_forward_lut_down_straddling_segments(moe):
    # down by table lookup with more (rank, chunk) segments (8 x 64) than
    # workgroups: 8 tiles per workgroup, so most ranges span two segments
    # and each combine polls 512 partials per row over several round trips
    _check_decode(moe, synth.get_config("mixtral", H=256, I=8192, E=16, k=8, tokens=2, layers=2), method="lookup",
                  down="lookup")


def test_decode_forward_lut_forced_k3_shape(moe, monkeypatch):
    # forced table lookup at the K3 slice shape (H 5120, I 2048, top-16 of
    # 768, shared expert): 320 output slices for 256 workgroups, so some
    # workgroups combine two slices
    monkeypatch.setenv("MOE_DECODE_LUT", "1")
    _check_decode(moe, synth.get_config("k3_slice", tokens=1, layers=2), method="lookup", down="lookup")


def test_decode_forward_lut_shared_sigmoid(moe, monkeypatch):
    # forced table lookup with a shared expert, sigmoid top-8 and Zipf bias
    monkeypatch.setenv("MOE_DECODE_LUT", "1")
    _check_decode(moe, synth.get_config("kimi_linear", H=2048, I=2048, E=64, tokens=2, layers=2), method="lookup",
                  down="lookup")


def _streamed_setup(moe, cfg, capacity, pageable=False):
    from routed_expert_streaming_amd.device_workload import DeviceWorkload, HostRecordPool
    dw = DeviceWorkload(cfg)                       # resident copy: the reference for transparency
    hp = HostRecordPool(cfg, list(range(cfg.layers)), pin_limit=0 if pageable else 52 << 30)
    assert hp.pinned_records == (0 if pageable else cfg.layers * cfg.E)
    pool = torch.empty(capacity * hp.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(capacity, hp.stride, pool)
    return dw, hp, cache


@pytest.mark.parametrize("capacity,pageable", [(16, False), (23, False), (40, False), (23, True)])
def test_streamed_trace_and_transparency(moe, capacity, pageable):
    # K3 structure with fewer experts so that a few tokens exercise hits,
    # misses and evictions at capacity == k and above; pageable: every record
    # in pageable host memory (copied through the cache's pinned bounce
    # buffers)
    cfg = synth.get_config("k3_slice", tokens=5, layers=2, E=48)
    dw, hp, cache = _streamed_setup(moe, cfg, capacity, pageable)
    x = dw.inputs()
    copy_stream = torch.cuda.Stream()
    outs, idxs = [], []
    tables = [hp.table(L) for L in range(cfg.layers)]
    ws = torch.empty(moe.streamed_workspace_bytes(dw.layers[0]), dtype=torch.uint8, device="cuda")
    for t in range(cfg.tokens):
        for L in range(cfg.layers):
            idx = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
            o = moe.layer_forward_streamed(dw.layers[L], cache, L, None, x[t, L][None].contiguous(), copy_stream,
                                           ws=ws, idx=idx, host_table=tables[L])
            outs.append(o.clone())
            idxs.append(idx.clone())
    torch.cuda.synchronize()
    # transparency: identical bits to the resident layer path (same kernels,
    # same partial-sum split, fixed combine order)
    for n, (o, i) in enumerate(zip(outs, idxs)):
        t, L = divmod(n, cfg.layers)
        ro, ri, _ = moe.layer_forward(dw.layers[L], x[t, L][None].contiguous())
        assert torch.equal(o[0], ro[0]), f"streamed != resident at token {t} layer {L}"
        assert torch.equal(i[0], ri[0])
    # trace: bit-exact against the oracle's LRU over the oracle's own routing
    x64 = x.cpu().numpy().astype(np.float64)
    oidx = np.zeros((cfg.tokens * cfg.layers, cfg.k), np.int32)
    for t in range(cfg.tokens):
        for L in range(cfg.layers):
            oidx[t * cfg.layers + L] = oracle.route(dw.wl.router(L), dw.wl.bias(L), x64[t, L][None], cfg.k,
                                                    cfg.score)[0][0]
    key, hit, slot, ev = oracle.stream_trace(oidx, cfg.layers, cfg.E, capacity)
    tr = cache.trace()
    assert [r[0] for r in tr] == key.tolist()
    assert [r[1] for r in tr] == hit.tolist()
    assert [r[2] for r in tr] == slot.tolist()
    assert [(-1 if r[3] is None else r[3]) for r in tr] == ev.tolist()
    st = cache.stats()
    log(f"streamed capacity={capacity}: hits {st['hits']}/{st['lookups']} evictions {st['evictions']}")
    cache.close()


def test_streamed_rejects_capacity_below_k(moe):
    cfg = synth.get_config("k3_slice", tokens=1, layers=1, E=32)
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    dw = DeviceWorkload(cfg, with_records=False)
    pool = torch.empty(8 * 12013568, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(8, 12013568, pool)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_forward_streamed(dw.layers[0], cache, 0, [1] * cfg.E, dw.inputs()[0, 0][None].contiguous(),
                                   torch.cuda.Stream())
    assert e.value.code == -1
    cache.close()


@pytest.mark.parametrize("threshold", [False, True])
def test_streamed_lookahead_chained(moe, threshold):
    # Chained decode (each layer reads the rescaled residual stream, so the
    # next layer's router applied to this layer's input predicts something):
    # the look-ahead changes which copies happen and when, never the outputs;
    # the cache trace (lookups and look-ahead touches) replays exactly through
    # the oracle's LRU; actual and predicted expert sets match the oracle's
    # routers wherever the top-k boundary is not a near-tie.  With a
    # confidence threshold (min_weight = 1 / k_ahead) only the predictions of
    # at least that renormalised weight are touched.
    from routed_expert_streaming_amd.device_workload import chain_next_input
    cfg = synth.get_config("k3_slice", tokens=4, layers=3, E=48)
    capacity, k_ahead = 40, cfg.k
    min_w = 1.0 / k_ahead if threshold else 0.0
    dw, hp, cache = _streamed_setup(moe, cfg, capacity)
    pool2 = torch.empty(capacity * hp.stride, dtype=torch.uint8, device="cuda")
    cache_plain = moe.ExpertCache(capacity, hp.stride, pool2)
    x = dw.inputs()
    copy_stream = torch.cuda.Stream()
    tables = [hp.table(L) for L in range(cfg.layers)]
    ws = torch.empty(moe.streamed_workspace_bytes(dw.layers[0]), dtype=torch.uint8, device="cuda")

    def run(mode):
        outs, ins = [], []
        for t in range(cfg.tokens):
            h = x[t, 0].clone()
            scale = h.pow(2).mean().sqrt()
            xin = x[t, 0][None].contiguous()
            for L in range(cfg.layers):
                ins.append(xin.clone())
                if mode == "resident":
                    o, _, _ = moe.layer_forward(dw.layers[L], xin)
                else:
                    ahead = None
                    if mode == "ahead" and L + 1 < cfg.layers:
                        ahead = (dw.layers[L + 1], L + 1, tables[L + 1], k_ahead, min_w)
                    c = cache if mode == "ahead" else cache_plain
                    o = moe.layer_forward_streamed(dw.layers[L], c, L, None, xin, copy_stream, ws=ws,
                                                   host_table=tables[L], ahead=ahead)
                outs.append(o.clone())
                xin = chain_next_input(h, o, scale)
        torch.cuda.synchronize()
        return outs, ins

    out_a, in_a = run("ahead")
    out_p, _ = run("plain")
    out_r, _ = run("resident")
    for n in range(len(out_a)):
        assert torch.equal(out_a[n], out_p[n]), f"look-ahead changed output {n}"
        assert torch.equal(out_a[n], out_r[n]), f"streamed != resident at {n}"
    # replay of the cache's own operation string through the oracle's LRU
    tr = cache.trace()
    keys = np.array([r[0] for r in tr], np.int64)
    hit, slot, ev = oracle.lru(keys, capacity)
    assert [int(r[1] in (1, 3)) for r in tr] == hit.tolist()
    assert [r[2] for r in tr] == slot.tolist()
    assert [(-1 if r[3] is None else r[3]) for r in tr] == ev.tolist()
    # operation string: per (t, L) k lookups, then k_ahead touches of L + 1
    pos, checked = 0, 0
    for t in range(cfg.tokens):
        for L in range(cfg.layers):
            n = t * cfg.layers + L
            x64 = in_a[n].cpu().numpy().astype(np.float64)
            look = tr[pos:pos + cfg.k]
            pos += cfg.k
            assert all(r[1] in (0, 1) for r in look)
            ridx, _, z = oracle.route(dw.wl.router(L), dw.wl.bias(L), x64, cfg.k, cfg.score)
            zs = np.sort(z[0])[::-1]
            if zs[cfg.k - 1] - zs[cfg.k] > 1e-4:
                assert sorted(r[0] - L * cfg.E for r in look) == sorted(ridx[0].tolist())
                checked += 1
            if L + 1 < cfg.layers:
                n_pred = 0
                while pos + n_pred < len(tr) and tr[pos + n_pred][1] in (2, 3):
                    n_pred += 1
                pred = tr[pos:pos + n_pred]
                pos += n_pred
                pidx, pw, zp = oracle.route(dw.wl.router(L + 1), dw.wl.bias(L + 1), x64, k_ahead, cfg.score)
                zs = np.sort(zp[0])[::-1]
                margin_ok = zs[k_ahead - 1] - zs[k_ahead] > 1e-4 and np.all(np.abs(pw[0] - min_w) > 1e-5)
                if margin_ok:
                    want = sorted(int(e) for e, w in zip(pidx[0], pw[0]) if w >= min_w)
                    assert sorted(r[0] - (L + 1) * cfg.E for r in pred) == want
                    checked += 1
    assert pos == len(tr) and checked >= len(out_a)
    st = cache.stats()
    assert st["ahead_inserted"] == sum(r[1] == 2 for r in tr)
    assert st["ahead_present"] == sum(r[1] == 3 for r in tr)
    assert st["ahead_used"] + st["ahead_wasted"] <= st["ahead_inserted"]
    assert st["lookups"] == sum(r[1] in (0, 1) for r in tr)
    log(f"look-ahead: {st}")
    cache.close()
    cache_plain.close()


def test_streamed_file_tier(moe, tmp_path):
    # Third tier: records in a file read with O_DIRECT into a small pinned
    # LRU pool behind a small HBM cache.  Outputs equal the resident path's
    # bit for bit; the host tier's trace replays exactly through the oracle's
    # LRU over the HBM misses in order; every tier miss is one record read.
    from routed_expert_streaming_amd.device_workload import DeviceWorkload, write_record_file
    cfg = synth.get_config("tiny", tokens=6, layers=3, E=16)
    path = str(tmp_path / "records.bin")
    stride = write_record_file(cfg, path, list(range(cfg.layers)))
    dw = DeviceWorkload(cfg)
    x = dw.inputs()
    hbm_slots, tier_slots = 4, 6
    pool = torch.empty(hbm_slots * stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(hbm_slots, stride, pool)
    tier = moe.HostTier(path, stride, cfg.layers * cfg.E, tier_slots, io_threads=3)
    copy_stream = torch.cuda.Stream()
    ws = torch.empty(moe.streamed_workspace_bytes(dw.layers[0]), dtype=torch.uint8, device="cuda")
    outs = []
    for t in range(cfg.tokens):
        for L in range(cfg.layers):
            o = moe.layer_forward_streamed(dw.layers[L], cache, L, None, x[t, L][None].contiguous(), copy_stream,
                                           ws=ws, tier=(tier, L * cfg.E))
            outs.append(o.clone())
    torch.cuda.synchronize()
    for n, o in enumerate(outs):
        t, L = divmod(n, cfg.layers)
        ro, _, _ = moe.layer_forward(dw.layers[L], x[t, L][None].contiguous())
        assert torch.equal(o[0], ro[0]), f"file tier != resident at token {t} layer {L}"
    misses = np.array([r[0] for r in cache.trace() if r[1] == 0], np.int64)   # key = layer * E + e = record
    tr = tier.trace()
    assert [r[0] for r in tr] == misses.tolist()
    hit, slot, ev = oracle.lru(misses, tier_slots)
    assert [r[1] for r in tr] == hit.tolist()
    assert [r[2] for r in tr] == slot.tolist()
    assert [(-1 if r[3] is None else r[3]) for r in tr] == ev.tolist()
    st = tier.stats()
    assert st["lookups"] == len(misses) and st["reads"] == len(misses) - int(hit.sum())
    assert st["read_bytes"] == st["reads"] * stride
    log(f"file tier: {st}, HBM misses {len(misses)} of {len(cache.trace())}")
    tier.close()
    cache.close()


def test_streamed_file_tier_exclusive(moe, tmp_path):
    # The file tier as the HBM cache's exclusive lower tier: an HBM miss is
    # looked up in host memory (a key found there leaves it), else read from
    # the file; the key the HBM cache evicts moves down, copied device to
    # host from its slot.  Outputs equal the resident path's bit for bit (a
    # record that went down and came back up carries the right bytes); the
    # HBM trace and the host tier's operation string equal the oracle's
    # two-tier model over the lookups in order; together the tiers hit
    # exactly where one LRU of their combined size hits.
    from routed_expert_streaming_amd.device_workload import DeviceWorkload, write_record_file
    cfg = synth.get_config("tiny", tokens=8, layers=3, E=16)
    path = str(tmp_path / "records.bin")
    stride = write_record_file(cfg, path, list(range(cfg.layers)))
    dw = DeviceWorkload(cfg)
    x = dw.inputs()
    hbm_slots, lower = 4, 6
    pool = torch.empty(hbm_slots * stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(hbm_slots, stride, pool)
    tier = moe.HostTier(path, stride, cfg.layers * cfg.E, lower + moe.MOE_MAX_K, io_threads=3, exclusive=True)
    copy_stream = torch.cuda.Stream()
    ws = torch.empty(moe.streamed_workspace_bytes(dw.layers[0]), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError):   # keys shared with the HBM cache: record0 = layer * E
        moe.layer_forward_streamed(dw.layers[1], cache, 1, None, x[0, 1][None].contiguous(), copy_stream, ws=ws,
                                   tier=(tier, 0))
    outs = []
    for t in range(cfg.tokens):
        for L in range(cfg.layers):
            o = moe.layer_forward_streamed(dw.layers[L], cache, L, None, x[t, L][None].contiguous(), copy_stream,
                                           ws=ws, tier=(tier, L * cfg.E))
            outs.append(o.clone())
    torch.cuda.synchronize()
    for n, o in enumerate(outs):
        t, L = divmod(n, cfg.layers)
        ro, _, _ = moe.layer_forward(dw.layers[L], x[t, L][None].contiguous())
        assert torch.equal(o[0], ro[0]), f"exclusive file tier != resident at token {t} layer {L}"
    ctr = cache.trace()
    keys = np.array([r[0] for r in ctr], np.int64)
    m = oracle.two_tier(keys, hbm_slots, lower)
    assert [r[1] for r in ctr] == m["hit1"].tolist()
    assert [r[2] for r in ctr] == m["slot1"].tolist()
    assert [(-1 if r[3] is None else r[3]) for r in ctr] == m["ev1"].tolist()
    want = []
    for i in range(len(keys)):
        if m["hit1"][i]:
            continue
        want.append((int(keys[i]), 1 if m["hit2"][i] else 4, int(m["slot2"][i]), -1))
        if m["ev1"][i] != -1:
            want.append((int(m["ev1"][i]), 5, int(m["dslot"][i]), int(m["dev"][i])))
    got = [(r[0], r[1], r[2], -1 if r[3] is None else r[3]) for r in tier.trace()]
    assert got == want
    both, _, _ = oracle.lru(keys, hbm_slots + lower)
    assert (((m["hit1"] == 1) | (m["hit2"] == 1)).astype(np.int32)).tolist() == both.tolist()
    st = tier.stats()
    n_miss = int((m["hit1"] == 0).sum())
    n_low = int((m["hit2"] == 1).sum())
    assert n_low > 0, "the run should find evicted records in host memory"
    assert st["lookups"] == n_miss and st["hits"] == n_low and st["reads"] == n_miss - n_low
    assert st["demotions"] == int((m["ev1"] != -1).sum())
    log(f"exclusive file tier: {st}, HBM misses {n_miss} of {len(keys)}, found below {n_low}")
    tier.close()
    cache.close()


# ---------------------------------------------------------------- routing edges
@pytest.mark.parametrize("k,score", [(1, "softmax"), (1, "sigmoid"), (8, "softmax"), (8, "sigmoid")])
def test_routing_edge_k(moe, k, score):
    # k = 1 (the weight is exactly 1) and k = E (every expert; softmax-renorm
    # is the full softmax): router, layer and decode kernels against the
    # oracle on the Tiny shape (8 experts); for k = 1 the router is redrawn
    # until every token's top-1 margin is at least 1e-3
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    cfg = synth.get_config("tiny", k=k, score=score)
    dw = DeviceWorkload(cfg)
    x = dw.inputs()[:, 0, :].contiguous()
    idx, w = moe.route_topk(dw.layers[0].router, x)
    x64 = x.cpu().numpy().astype(np.float64)
    ridx, rw, z = oracle.route(dw.wl.router(0), None, x64, k, score)
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    if k == 1:
        assert np.array_equal(idx, ridx)
        assert np.all(w == 1.0)
    else:
        assert np.array_equal(np.sort(idx, 1), np.tile(np.arange(cfg.E), (cfg.tokens, 1)))
        full = np.exp(z - z.max(1, keepdims=True)) if score == "softmax" else 1.0 / (1.0 + np.exp(-z))
        full = full / full.sum(1, keepdims=True)
        np.testing.assert_allclose(weights_by_expert(idx, w), full, rtol=2e-6, atol=1e-7)
        np.testing.assert_allclose(weights_by_expert(ridx, rw), full, rtol=1e-12)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-6)
    out, lidx, _ = moe.layer_forward(dw.layers[0], x)
    ref, _, _ = _oracle_layer(dw, 0, x64)
    assert same_sets(lidx.cpu().numpy(), ridx)
    r = rel_l2(out.cpu().numpy(), ref)
    log(f"k={k} {score}: layer rel_l2 {r:.3e}")
    assert r <= RTOL_F32_PATH
    _check_decode(moe, cfg)


# ----------------------------------------------------------------- fp16 range
def _scaled_layers(dw, sx, outlier_cols, so):
    """Layers whose experts see x * 2^sx (columns outlier_cols a further
    2^so) while the logits stay those of the unscaled input: the router
    weights are scaled by the inverse powers of two, so every fp32 product
    of the logit sums is the unscaled one exactly."""
    from routed_expert_streaming_amd import Layer, Router
    cfg = dw.cfg
    col = np.full(cfg.H, 2.0 ** sx)
    col[outlier_cols] *= 2.0 ** so
    layers, Ws = [], []
    for i, L in enumerate(dw.layer_ids):
        W = (dw.wl.router(L).astype(np.float64) / col).astype(np.float32)
        Ws.append(W)
        base = dw.layers[i]
        r = Router(torch.from_numpy(W).cuda(), cfg.k, cfg.score, base.router.bias)
        layers.append(Layer(cfg.H, cfg.I, r, shared=base.shared, record_ptrs=base.record_ptrs))
    return layers, Ws, torch.from_numpy(col.astype(np.float32)).cuda()


@pytest.mark.parametrize("name,lut", [("mixtral", None), ("mixtral", "0"), ("mixtral", "2"), ("k3_slice", None)])
def test_decode_fp16_range(moe, monkeypatch, name, lut):
    # activations far beyond fp16's range (|x| up to ~2^22, so |h| and the
    # table entries C[c].x_q would overflow 65504 without range scaling):
    # every decode method must stay finite and match the oracle
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    if lut is not None:
        monkeypatch.setenv("MOE_DECODE_LUT", lut)
    cfg = synth.get_config(name, tokens=2, layers=2)
    dw = DeviceWorkload(cfg)
    layers, Ws, col = _scaled_layers(dw, 15, np.arange(5, cfg.H, 97), 5)
    x = (dw.inputs() * col).contiguous()
    assert x.abs().max().item() > 65504.0 * 16
    out, idx = moe.decode_forward(layers, x)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    assert np.all(np.isfinite(out))
    oracle.set_threads(16)
    x64 = x.cpu().numpy().astype(np.float64)
    empty = np.zeros(1, np.uint8)
    worst = 0.0
    for t in range(cfg.tokens):
        for L in range(cfg.layers):
            ridx, _, _ = oracle.route(Ws[L], dw.wl.bias(L), x64[t, L][None], cfg.k, cfg.score)
            need = set(int(e) for e in ridx[0])
            recs = [dw.wl.record(L, e) if e in need else empty for e in range(cfg.E)]
            ref, ridx, _ = oracle.layer(Ws[L], dw.wl.bias(L), cfg.k, cfg.score, recs, dw.wl.shared(L), cfg.H, cfg.I,
                                        x64[t, L][None])
            assert same_sets(idx[t, L][None], ridx)
            r = rel_l2(out[t, L], ref[0])
            worst = max(worst, r)
            assert r <= RTOL_F32_PATH, f"token {t} layer {L}: rel_l2 {r:.3e}"
    log(f"{name} decode (MOE_DECODE_LUT={lut}) with |x| up to {np.abs(x64).max():.3g}: worst rel_l2 {worst:.3e}")


@pytest.mark.parametrize("name,T", [("k3_slice", 2), ("mixtral", 1)])
def test_layer_fp16_range(moe, name, T):
    # the multi-kernel layer path (also the streamed path's kernels) with the
    # same out-of-range activations
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    cfg = synth.get_config(name, tokens=T, layers=1)
    dw = DeviceWorkload(cfg, layers=[0])
    layers, Ws, col = _scaled_layers(dw, 15, np.arange(3, cfg.H, 89), 5)
    x = (dw.inputs()[:, 0, :] * col).contiguous()
    out, idx, _ = moe.layer_forward(layers[0], x)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    x64 = x.cpu().numpy().astype(np.float64)
    ridx, _, _ = oracle.route(Ws[0], dw.wl.bias(0), x64, cfg.k, cfg.score)
    need = set(int(e) for e in ridx.reshape(-1))
    empty = np.zeros(1, np.uint8)
    recs = [dw.wl.record(0, e) if e in need else empty for e in range(cfg.E)]
    oracle.set_threads(16)
    ref, ridx, _ = oracle.layer(Ws[0], dw.wl.bias(0), cfg.k, cfg.score, recs, dw.wl.shared(0), cfg.H, cfg.I, x64)
    assert same_sets(idx.cpu().numpy(), ridx)
    for t in range(T):
        r = rel_l2(out[t], ref[t])
        log(f"{name} layer token {t} with |x| up to {np.abs(x64).max():.3g}: rel_l2 {r:.3e}")
        assert r <= RTOL_F32_PATH
