"""The streaming-read reference kernels (measurement support) compute what
they claim: each written piece is the XOR of the slice's 16-byte pieces that
its lane read, for both launch shapes and a ragged slice length."""
import numpy as np
import pytest
import torch

from recurrent_state_quant_lq_amd import lq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("slice_bytes,n,write", [(28224, 37, 1536), (4096, 5, 4096), (65536, 3, 16),
                                                 (16, 9, 16), (30000 - 30000 % 16, 300, 0)])
@pytest.mark.parametrize("mode", [0, 1])
def test_stream_read_sink(slice_bytes, n, write, mode):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator(device="cuda").manual_seed(slice_bytes + n)
    src = torch.randint(0, 256, (n * slice_bytes,), dtype=torch.uint8, device="cuda", generator=g)
    sink = torch.zeros((max(1, n * write),), dtype=torch.uint8, device="cuda")
    lq.lq_measure_stream_read(src, slice_bytes, n, mode, 7, sink if write else None, write)
    torch.cuda.synchronize()
    if not write:
        return
    pieces = src.cpu().numpy().view(np.uint32).reshape(n, slice_bytes // 16, 4)
    nv = slice_bytes // 16
    want = np.zeros((n, 256, 4), np.uint32)
    for e in range(nv):
        want[:, e % 256] ^= pieces[:, e]
    got = sink.cpu().numpy().view(np.uint32).reshape(n, write // 16, 4)
    assert (got == want[:, :write // 16]).all()
