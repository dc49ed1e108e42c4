"""The stream-read probe (a measurement aid the bench uses for the HBM stream-read ceiling) reads every byte
of its buffer once (needs an MI355X): the XOR of its per-workgroup sink words is the XOR of every 32-bit word
of the buffer, whatever the grid."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 3 * 1024 * 1024 + 48, 64 * 1024 * 1024])
def test_stream_read_reads_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(-2**31, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    for config in range(la.stream_read_configs()):
        sink = la.stream_read(buf, config)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, (nbytes, config)
