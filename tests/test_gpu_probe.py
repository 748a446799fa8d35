"""The streaming probes that measure the device's HBM read and copy rates
(context for the roofline fractions, not part of the attention path): the
read probe must touch every byte once (its XOR of all 32-bit words equals the
host's), the copy probe must copy exactly the requested bytes, at grid sizes
that leave ragged tails.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_bf16_amd as da
from gpu_util import announce

pytestmark = pytest.mark.gpu


def host_xor(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.view(np.uint32)))


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 12345, (1 << 22) + 48])
@pytest.mark.parametrize("blocks,depth", [(1, 4), (7, 8), (0, 16), (0, 8), (300, 4)])
def test_read_probe_touches_every_word(nbytes, blocks, depth):
    announce(f"probe read bytes={nbytes} blocks={blocks} depth={depth}")
    rng = np.random.default_rng(nbytes + blocks)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    da.probe_stream_read(src, sink, blocks, depth)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == host_xor(host)
    # a second call XORs into the sink again: back to zero
    da.probe_stream_read(src, sink, blocks, depth)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0


@pytest.mark.parametrize("nbytes", [16, 16 * 12345, (1 << 22) + 48])
@pytest.mark.parametrize("blocks,depth", [(1, 4), (3, 8), (0, 16), (0, 4)])
def test_copy_probe_copies_exactly(nbytes, blocks, depth):
    announce(f"probe copy bytes={nbytes} blocks={blocks} depth={depth}")
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    guard = 256
    dst = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    da.probe_stream_copy(src, dst[:nbytes], blocks, depth)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())


def test_probes_reject_bad_arguments_with_real_buffers():
    src = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = da.lib()
    p = src.data_ptr()
    assert L.da_probe_stream_read(p, 24, 0, 8, sink.data_ptr(), None) == 1
    assert L.da_probe_stream_read(p + 4, 512, 0, 8, sink.data_ptr(), None) == 1
    assert L.da_probe_stream_read(p, 512, 0, 5, sink.data_ptr(), None) == 1
    assert L.da_probe_stream_copy(p, p + 256, 512, 0, 4, None) == 1
    with pytest.raises(ValueError):
        da.probe_stream_copy(src, src[:512])
