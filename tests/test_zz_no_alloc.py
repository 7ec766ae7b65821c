"""moe_decode_forward_noalloc (the decode driver with its workspace in the
library's own device scratch array, for callers that cannot allocate) against
moe_decode_forward with a caller workspace: identical outputs and expert ids,
bit for bit, on two calls in a row (the second smaller, after a different
shape has used the scratch), the status read through moe_decode_status(NULL),
and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_streaming_amd as m
    m.lib()
    return m


def _pair(moe, dw, x):
    ref_out, ref_idx = moe.decode_forward(dw.layers, x)
    out, idx = moe.decode_forward_noalloc(dw.layers, x)
    torch.cuda.synchronize()
    assert not moe.decode_status(None), "no-alloc decode hit its wait limit"
    return ref_out, ref_idx, out, idx


@pytest.mark.parametrize("first,second", [
    (("mixtral", dict(tokens=3, layers=4)), ("mixtral", dict(tokens=1, layers=2))),
    (("k3_slice", dict(tokens=2, layers=2)), ("kimi_linear", dict(tokens=2, layers=2))),
])
def test_noalloc_matches_workspace_path(moe, first, second):
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    for name, kw in (first, second):
        cfg = synth.get_config(name, **kw)
        log(f"no-alloc decode {name} {kw}")
        dw = DeviceWorkload(cfg)
        x = dw.inputs()
        ref_out, ref_idx, out, idx = _pair(moe, dw, x)
        assert torch.equal(idx, ref_idx), f"{name}: expert ids differ"
        assert torch.equal(out, ref_out), f"{name}: outputs differ"
        del dw
        torch.cuda.empty_cache()


def test_noalloc_rejects_beyond_scratch(moe):
    # a shape whose decode workspace exceeds the scratch array (Mixtral's
    # hidden and intermediate sizes with 6 experts per token: 34 MB of
    # table-lookup partials): rejected on the host with MOE_E_SPACE before
    # anything is launched (no records needed)
    from routed_expert_streaming_amd import Layer, Router
    H, I, E, k = 4096, 14336, 8, 6
    W = torch.zeros((E, H), dtype=torch.float32, device="cuda")
    layer = Layer(H, I, Router(W, k, "softmax"), record_ptrs=torch.zeros(E, dtype=torch.int64, device="cuda"))
    need = moe.decode_workspace_bytes([layer])
    assert need > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, 1, H), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.decode_forward_noalloc([layer], x)
    assert e.value.code == -3
