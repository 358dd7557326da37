"""The bandwidth probe used by the benchmark reads every word of its buffer:
its sink equals the XOR of all 32-bit words (computed on the host), for a
whole number of grid strides, a ragged tail and a buffer smaller than one
workgroup's share."""
import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
from tests.gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 2048 * 256 * 8 * 16, 3 * (1 << 24) + 16 * 7])
def test_stream_read_reads_every_word(nbytes):
    print(f"stream_read {nbytes} bytes", flush=True)
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(DEV)
    sink = spffn.stream_read(buf)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(want)
