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


def _lds_gather_expected(width, reps):
    """The LDS probe's sink recomputed on the host from its documented definition."""
    nwg, threads, chains = 256, 1024, 8
    gid = np.arange(nwg * threads, dtype=np.uint64)
    x = ((gid[:, None] * chains + np.arange(chains, dtype=np.uint64)) & 0xFFFFFFFF).astype(np.uint64)
    words = ((np.arange(32768, dtype=np.uint64) * 2654435761) & 0xFFFFFFFF).astype(np.uint32)
    bits = int(np.log2(131072 // width))
    acc = np.zeros(nwg * threads, np.uint32)
    for _ in range(reps):
        x = (x * 1664525 + 1013904223) & 0xFFFFFFFF
        idx = (x >> (32 - bits)).astype(np.int64)
        if width == 2:
            v = (words[idx >> 1] >> (16 * (idx & 1)).astype(np.uint32)) & 0xFFFF
        else:
            per = width // 4
            v = np.zeros_like(idx, dtype=np.uint32)
            for w in range(per):
                v ^= words[idx * per + w]
        acc ^= np.bitwise_xor.reduce(v.astype(np.uint32), axis=1)
    return np.bitwise_xor.reduce(acc.reshape(nwg, threads), axis=1)


@pytest.mark.parametrize("width", [2, 4, 8, 16])
def test_lds_gather_probe_reads_what_it_says(width):
    """The LDS random-gather probe (the bench's roof for batched lookups) performs exactly the lookups its
    definition lists: its per-workgroup sink equals the host's recomputation."""
    sink = la.lds_gather(width, 3)
    torch.cuda.synchronize()
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), _lds_gather_expected(width, 3))
