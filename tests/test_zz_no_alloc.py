"""rq_lut_logits_static, the head call for callers that cannot allocate: it runs on the library's own
per-GPU scratch array and must give exactly what rq_lut_logits gives with a caller's workspace (same
kernels, same plan), call after call, whatever the previous call left in the scratch."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
from lut_logits_amd import binding as B
from lut_logits_amd import synth
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


def _both(W, h, softcap, topk, lut_dtype="f32"):
    lut = la.build_lut(W, dev(h), lut_dtype=lut_dtype)
    Bn = h.shape[0]
    ref = la.lut_logits(W, lut, Bn, softcap=softcap, topk=topk)
    got = la.lut_logits_static(W, lut, Bn, softcap=softcap, topk=topk)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got):
    for a, b in zip(ref, got):
        assert (a is None) == (b is None)
        if a is not None:
            assert torch.equal(a, b)


def test_static_matches_workspace_twice_then_smaller():
    """Two calls in a row, the second on a smaller head: the Gemma-2-2B head at B=1 with top-50 (4.2 MB of
    scratch, G=4 partial sums), then the tiny head with top-5 at B=2 (G=1, other offsets in the scratch). Each
    equals rq_lut_logits bit for bit, and a third call repeats the first one's bits."""
    cfg = synth.CONFIGS["gemma_b1"]
    mat, h, _ = synth.make_head(cfg)
    Wg = to_dev(mat)
    ref1, got1 = _both(Wg, h, cfg.softcap, 50)
    _same(ref1, got1)
    tiny = synth.CONFIGS["tiny"]
    tmat, _, _ = synth.make_head(tiny)
    th = synth.gen_hidden(np.random.default_rng(9), 2, tiny.D)
    Wt = to_dev(tmat)
    ref2, got2 = _both(Wt, th, tiny.softcap, 5)
    _same(ref2, got2)
    lut = la.build_lut(Wg, dev(h))
    again = la.lut_logits_static(Wg, lut, 1, softcap=cfg.softcap, topk=50)
    _same(got1, again)


def test_static_argmax_only_and_bf16_table():
    """No logits output (a logits scratch inside the static array for the top-k) and a bf16 table."""
    mat, h = synth.gen_exact(61, 3000, 96, 16, 256, 2, 3)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h), lut_dtype="bf16")
    ref = la.lut_logits(W, lut, 3, softcap=30.0, logits=False, topk=7)
    got = la.lut_logits_static(W, lut, 3, softcap=30.0, logits=False, topk=7)
    _same(ref, got)


def test_static_refuses_calls_beyond_its_scratch():
    """A call needing more than RQ_STATIC_SCRATCH_BYTES (the Gemma head at B=16: 33 MB of partial sums)
    returns RQ_ERR_WORKSPACE and writes nothing."""
    cfg = synth.CONFIGS["gemma_b16"]
    mat, h, _ = synth.make_head(cfg, V=256000)
    W = to_dev(mat)
    assert la.lut_logits_workspace(W, 16) > (16 << 20)
    lut = torch.zeros(la.lut_bytes(W, 16) // 4, dtype=torch.float32, device="cuda")
    out = torch.full((16, W.rows), 7.0, device="cuda")
    with pytest.raises(B.RQError) as e:
        la.lut_logits_static(W, lut, 16, out=out)
    assert e.value.status == B.RQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
