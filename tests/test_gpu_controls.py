"""The bandwidth controls a measurement runs beside the codec kernels (streaming copy, read and
fill), checked for their results on the GPU at sizes that leave ragged passes: the copy equals
its source, the read's XOR fold equals numpy's, the fill writes every word and nothing past
the end."""
import numpy as np
import pytest
import torch

from kv_cache_compression_vector_amd import kvq
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SIZES = [16, 16 * 1023, 16 * 1025, 16 * 262147, 16 * (1 << 22) + 16 * 77]


def _words(n16, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(-(1 << 31), (1 << 31) - 1, (4 * n16,), generator=g, device=DEV,
                         dtype=torch.int32)


@pytest.mark.parametrize("nbytes", SIZES)
def test_stream_copy_read_fill(nbytes):
    say(f"stream controls bytes={nbytes}")
    n16 = nbytes // 16
    src = _words(n16, 11 + n16)
    dst = torch.zeros(4 * n16 + 8, dtype=torch.int32, device=DEV)  # 32 guard bytes
    kvq.stream_copy(dst[:4 * n16], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:4 * n16], src)
    assert int(dst[4 * n16:].abs().sum()) == 0
    sink = torch.tensor([0x5A5A5A5A], dtype=torch.int32, device=DEV)
    kvq.stream_read(src, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32)) ^ np.uint32(0x5A5A5A5A)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    kvq.stream_fill(dst[:4 * n16], 0xC0FFEE11)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    assert (got[:4 * n16] == 0xC0FFEE11).all()
    assert (got[4 * n16:] == 0).all()
