"""The C-ABI library loads and exports every symbol include/moe.h declares;
host-side argument validation (no kernel is launched by these calls)."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from routed_expert_streaming_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from routed_expert_streaming_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:moe|expert_cache)_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(L, n), n
    from routed_expert_streaming_amd import _lib
    assert set(names) == set(_lib.SIGNATURES)


def test_abi_version(L):
    assert L.moe_abi_version() == 1


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_record_layout_matches_format(L, name):
    from routed_expert_streaming_amd import _lib
    cfg = synth.CONFIGS[name]
    out = _lib.MoeRecordLayout()
    assert L.moe_rvq_record_layout(cfg.H, cfg.I, ctypes.byref(out)) == 0
    lay = synth.record_layout(cfg.H, cfg.I)
    assert tuple(out.offset) == lay.offsets and tuple(out.size) == lay.sizes
    assert (out.nbytes, out.padded) == (lay.nbytes, lay.padded)


def test_record_layout_rejects_bad_dims(L):
    from routed_expert_streaming_amd import _lib
    out = _lib.MoeRecordLayout()
    for H, I in ((200, 512), (256, 100), (0, 128), (-128, 128)):
        assert L.moe_rvq_record_layout(H, I, ctypes.byref(out)) == _lib.MOE_E_INVAL
    assert L.moe_rvq_record_layout(256, 512, None) == _lib.MOE_E_INVAL


def _layer(E=8, k=2, H=256, I=512, score=0, weight=1, records=1):
    from routed_expert_streaming_amd import _lib
    return _lib.MoeLayer(H, I, _lib.MoeRouter(weight, None, E, k, score), records, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(k=0), b"k=0"), (dict(k=9), b"k=9"), (dict(E=2000, k=2), b"E=2000"), (dict(k=33, E=64), b"k=33"),
    (dict(H=200), b"multiples of 128"), (dict(I=100), b"multiples of 128"), (dict(score=7), b"score_fn"),
    (dict(weight=None), b"router weight"), (dict(records=None), b"records"),
])
def test_layer_forward_validation(L, kw, needle):
    from routed_expert_streaming_amd import _lib
    lay = _layer(**kw)
    rc = L.moe_layer_forward(ctypes.byref(lay), 1, 0, 1, 1, None, None, 1, 1 << 30, None)
    assert rc == _lib.MOE_E_INVAL
    assert needle in L.moe_last_error()


def test_layer_forward_workspace_too_small(L):
    from routed_expert_streaming_amd import _lib
    lay = _layer()
    need = L.moe_layer_workspace_bytes(ctypes.byref(lay), 4)
    assert need > 0
    rc = L.moe_layer_forward(ctypes.byref(lay), 1, 0, 4, 1, None, None, 1, need - 1, None)
    assert rc == _lib.MOE_E_SPACE


def test_zero_tokens_noop_and_bad_dtype(L):
    from routed_expert_streaming_amd import _lib
    lay = _layer()
    assert L.moe_layer_forward(ctypes.byref(lay), None, 0, 0, None, None, None, None, 0, None) == 0
    assert L.moe_layer_forward(ctypes.byref(lay), 1, 5, 1, 1, None, None, 1, 1 << 30, None) == _lib.MOE_E_INVAL


def test_ffn_validation(L):
    from routed_expert_streaming_amd import _lib
    assert L.moe_expert_ffn_rvq(None, 256, 512, 1, 1, None, 1, 0, 1, 1 << 30, None) == _lib.MOE_E_INVAL
    assert L.moe_expert_ffn_rvq(0x1001, 256, 512, 1, 1, None, 1, 0, 1, 1 << 30, None) == _lib.MOE_E_INVAL
    assert b"256-byte" in L.moe_last_error()
    assert L.moe_expert_ffn_rvq(0x1000, 256, 500, 1, 1, None, 1, 0, 1, 1 << 30, None) == _lib.MOE_E_INVAL


def test_decode_validation(L):
    from routed_expert_streaming_amd import _lib
    arr = (_lib.MoeLayer * 2)(_layer(), _layer(I=1024))
    rc = L.moe_decode_forward(arr, 2, 1, 1, 1, None, 1, 1 << 30, None)
    assert rc == _lib.MOE_E_INVAL and b"differs" in L.moe_last_error()


def test_cache_create_validation(L):
    from routed_expert_streaming_amd import _lib
    h = ctypes.c_void_p()
    assert L.expert_cache_create(0, 4096, 1, ctypes.byref(h)) == _lib.MOE_E_INVAL
    assert L.expert_cache_create(4, 100, 1, ctypes.byref(h)) == _lib.MOE_E_INVAL
    assert L.expert_cache_create(4, 4096, None, ctypes.byref(h)) == _lib.MOE_E_INVAL
    assert L.expert_cache_lookup(None, 1, ctypes.byref(ctypes.c_int32())) == _lib.MOE_E_INVAL


def test_host_tier_rejects_bad_arguments(L, tmp_path):
    # argument checks that run before any HIP call (no GPU needed)
    from routed_expert_streaming_amd._lib import MOE_E_INVAL
    h = ctypes.c_void_p()
    f = tmp_path / "r.bin"
    f.write_bytes(b"\0" * 8192)
    pool = ctypes.create_string_buffer(3 * 4096 + 4096)
    aligned = (ctypes.addressof(pool) + 4095) & ~4095
    assert L.moe_host_tier_create(str(f).encode(), 4000, 2, 1, aligned, 1, ctypes.byref(h)) == MOE_E_INVAL
    assert L.moe_host_tier_create(str(f).encode(), 4096, 2, 1, aligned + 16, 1, ctypes.byref(h)) == MOE_E_INVAL
    assert L.moe_host_tier_create(str(tmp_path / "none").encode(), 4096, 2, 1, aligned, 1, ctypes.byref(h)) == \
        MOE_E_INVAL
    assert L.moe_host_tier_create(str(f).encode(), 4096, 3, 1, aligned, 1, ctypes.byref(h)) == MOE_E_INVAL   # short
    assert L.moe_host_tier_create(str(f).encode(), 4096, 2, 0, aligned, 1, ctypes.byref(h)) == MOE_E_INVAL
    assert L.moe_host_tier_create(str(f).encode(), 4096, 2, 1, aligned, 0, ctypes.byref(h)) == MOE_E_INVAL
    assert not h.value


def test_hbm_read_validation(L):
    # rejected before any device call
    from routed_expert_streaming_amd import _lib
    sink = ctypes.c_void_p(4096)
    assert L.moe_hbm_read(None, 16, sink, None) == _lib.MOE_E_INVAL
    assert L.moe_hbm_read(ctypes.c_void_p(4096), 16, None, None) == _lib.MOE_E_INVAL
    assert L.moe_hbm_read(ctypes.c_void_p(4104), 16, sink, None) == _lib.MOE_E_INVAL   # not 16-byte aligned
    assert L.moe_hbm_read(ctypes.c_void_p(4096), 24, sink, None) == _lib.MOE_E_INVAL   # not a multiple of 16


@pytest.mark.parametrize("fn", ["moe_decode_gate_up_method", "moe_decode_down_method"])
def test_decode_method_queries_reject_bad_arguments(L, fn):
    m = ctypes.c_int32(-1)
    assert getattr(L, fn)(None, 1, ctypes.byref(m)) == -1
    assert getattr(L, fn)(None, 0, None) == -1
    assert m.value == -1
