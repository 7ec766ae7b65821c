"""The plain-read reference kernel (moe_hbm_read) that bench.py times beside
the decode: every 32-bit word of the buffer is read exactly once (the XOR of
its partials equals the XOR of the words; a skipped or doubled word breaks
it), for sizes below, at and well above one grid stride, with ragged tails."""
import numpy as np
import pytest
import torch

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routed_expert_streaming_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, 2048 * 256 * 16, 2048 * 256 * 16 * 4 + 7 * 16,
                                    (48 << 20) + 16 * 1000])
def test_hbm_read_reads_every_word_once(moe, nbytes):
    log(f"hbm_read {nbytes} bytes")
    rng = np.random.default_rng(nbytes + 1)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = moe.hbm_read(buf)
    torch.cuda.synchronize()
    parts = sink.cpu().numpy().view(np.uint32)
    assert parts.shape == (moe.HBM_READ_BLOCKS,)
    want = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert np.bitwise_xor.reduce(parts) == want
    if nbytes == 0:
        assert not parts.any()
