"""Synthetic workload generator: determinism, margins, formats, byte counts."""
import numpy as np
import torch

import synth


def test_records_deterministic_and_distinct():
    cfg = synth.CONFIGS["tiny"]
    a = synth.make_record(cfg, 0, 1)
    assert np.array_equal(a, synth.make_record(cfg, 0, 1))
    assert not np.array_equal(a, synth.make_record(cfg, 0, 2))
    lay = synth.record_layout(cfg.H, cfg.I)
    assert np.all(a[lay.nbytes:] == 0)               # padding is zero


def test_fill_records_parallel_matches_serial():
    cfg = synth.CONFIGS["tiny"]
    wl = synth.Workload(cfg)
    keys = [(0, e) for e in range(cfg.E)]
    bufs = [np.empty(wl.layout.padded, np.uint8) for _ in keys]
    wl.fill_records(keys, bufs, threads=4)
    for (L, e), b in zip(keys, bufs):
        assert np.array_equal(b, synth.make_record(cfg, L, e))


def test_tiny_router_meets_margin():
    cfg = synth.CONFIGS["tiny"]
    wl = synth.Workload(cfg)
    m = synth.topk_margins(wl.router(0), None, wl.inputs()[:, 0, :], cfg.k)
    assert np.all(m >= synth.MARGIN)


def test_decode_inputs_meet_margin_after_redraw():
    cfg = synth.get_config("k3_slice", tokens=24, layers=3)
    wl = synth.Workload(cfg)
    x = wl.inputs()
    for L in range(cfg.layers):
        m = synth.topk_margins(wl.router(L), wl.bias(L), x[:, L, :], cfg.k)
        assert np.all(m >= synth.MARGIN)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), ref)


def test_batched_inputs_are_bf16_values():
    cfg = synth.get_config("batched", tokens=8)
    x = synth.Workload(cfg).inputs()
    assert np.array_equal(synth.bf16_bits_to_f32(synth.to_bf16_bits(x)), x)


def test_zipf_bias_ranks():
    cfg = synth.CONFIGS["kimi_linear"]
    b = synth.make_bias(cfg, 3)
    s = np.sort(b)[::-1]
    beta = 0.5 * 0.05 * np.sqrt(cfg.H)
    np.testing.assert_allclose(s, -1.1 * beta * np.log(np.arange(1, cfg.E + 1)), rtol=1e-6, atol=1e-6)


def test_expert_bytes_per_token():
    assert synth.expert_bytes_per_token(synth.CONFIGS["mixtral"]) == 4_244_635_648
    assert synth.expert_bytes_per_token(synth.CONFIGS["kimi_linear"]) == 999_862_272
    assert synth.expert_bytes_per_token(synth.CONFIGS["k3_slice"]) == 2_040_791_040
    assert synth.CONFIGS["k3_slice"].cache_capacity == 1536
