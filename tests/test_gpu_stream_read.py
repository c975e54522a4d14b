"""GPU check of the streaming-read measurement call (bw_stream_read): every byte
is read once, quarter by quarter (the XOR of each 4 KB quarter of a 16 KB
block's 32-bit words)."""
import numpy as np
import pytest
import torch

import ternary_weight_bit_amd as bw
from tests.gpu_helpers import host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16384, 16384 * 5 + 48, 12_582_912])
def test_block_xor(nbytes):
    rs = np.random.default_rng(nbytes)
    a = rs.integers(0, 256, size=nbytes, dtype=np.uint8)
    sink = host(bw.bw_stream_read(torch.from_numpy(a).to("cuda:0"))).view(np.uint32)
    pad = np.zeros((-nbytes) % 16384, np.uint8)
    ref = np.bitwise_xor.reduce(np.concatenate([a, pad]).view("<u4").reshape(-1, 1024), axis=1)
    assert np.array_equal(sink, ref)
