"""The per-token decode loop (lut_logits_amd.composite) against the oracle, token by token (needs an MI355X).

The loop feeds each argmax back as the next token on the device. The oracle is run teacher-forced: for
every step it takes the token the GPU chose, rebuilds that token's embedding row, the sqrt(D) scale, the
blocks (fp64) on the GPU's inputs to them and the head, and the GPU's blocks and next token must agree
with it."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
import oracle
from lut_logits_amd import synth
from lut_logits_amd.composite import DecodeLoop
from gpu_util import check_logits, host, to_dev

pytestmark = pytest.mark.gpu

O = oracle.default


def _rms(v):
    v = np.asarray(v, np.float64)
    return v / np.sqrt((v * v).mean(axis=-1, keepdims=True) + 1e-6)


def check_loop_step(o, head, layers, loop, tok, softcap):
    """One step of the loop, teacher-forced: every block's GPU output against the oracle's block on the
    GPU's input to it, the norms and residual stream (rq_residual_norm) against numpy to fp32 rounding, and the
    next token within 2t of the oracle head's maximum on the GPU's final hidden vector. Returns it."""
    row, _ = o.decode_rows(head.codes, head.codebooks, head.cb_is_bf16, np.array([tok], np.int32), False)
    h = row.astype(np.float64) * np.sqrt(head.D)
    for i, (gate, up, down) in enumerate(layers):
        x = host(loop.ins[i])
        assert np.allclose(x, _rms(h), rtol=0, atol=1e-5 * np.abs(_rms(h)).max()), f"block {i}: pre-norm"
        _, _, _, oy = o.mlp(*((m.codes, m.codebooks, False) for m in (gate, up, down)), x)
        y = host(loop.outs[i])
        check_logits(y, oy)
        h = h + _rms(y)
    last = host(loop.last)
    assert np.allclose(last, _rms(h), rtol=0, atol=1e-4 * np.abs(_rms(h)).max()), "final norm"
    _, ref = o.logits(head.codes, head.codebooks, head.cb_is_bf16, last, softcap)
    assert np.isfinite(ref).all()
    return ref


def test_decode_loop_teacher_forced():
    cfg = synth.CONFIGS["tiny"]
    head, _, _ = synth.make_head(cfg)
    rng = np.random.default_rng(11)
    hid, inter, d, K = cfg.D, 160, 2, 64
    layers = []
    for _ in range(3):
        gate = synth.gen_matrix(rng, inter, hid, hid // d, K, 2, (0.02, 0.005), "f32")
        up = synth.gen_matrix(rng, inter, hid, hid // d, K, 2, (0.02, 0.005), "f32")
        down = synth.gen_matrix(rng, hid, inter, inter // d, K, 2, (0.02, 0.005), "f32")
        layers.append((gate, up, down))
    Wh = to_dev(head)
    loop = DecodeLoop(Wh, [tuple(to_dev(m) for m in lay) for lay in layers], softcap=cfg.softcap, max_tokens=8,
                      keep_layers=True)
    loop.ids[0] = 7
    o = O()
    tokens = [7]
    for t in range(8):
        loop.step(t)
        nxt = int(loop.ids[t + 1].item())
        ref = check_loop_step(o, head, layers, loop, tokens[-1], cfg.softcap)
        tol = 1e-5 * np.abs(ref).max()
        assert ref[0, nxt] >= ref[0].max() - 2 * tol, f"step {t}: token {nxt} is not a maximum of the oracle"
        tokens.append(nxt)
    assert torch.equal(loop.ids[:9].cpu(), torch.tensor(tokens, dtype=torch.int32))
    # a second run from the same token repeats the sequence (deterministic)
    ids2 = loop.run(7, 8).clone()
    assert torch.equal(ids2.cpu(), torch.tensor(tokens, dtype=torch.int32))


@pytest.mark.parametrize("D", [1, 7, 1023, 1025, 2304, 9216, 70001])
def test_residual_norm_against_numpy(D):
    """rq_residual_norm: h += rms(y), x = rms(h), against the fp64 definition (rms(v) = v / sqrt(mean(v^2)
    + eps)): fp32 rounding only, over lengths below, at and past one element per thread and several per
    thread; without y it only normalises; h and x are distinct buffers and nothing else is written."""
    rng = np.random.default_rng(D)
    h0 = (rng.standard_normal(D) * 3.0).astype(np.float32)
    y0 = (rng.standard_normal(D) * 0.5 + 0.1).astype(np.float32)
    h = torch.from_numpy(h0.copy()).cuda()
    y = torch.from_numpy(y0.copy()).cuda()
    x = torch.full((D + 64,), 7.0, device="cuda")
    la.residual_norm(h, x[:D], y, eps=1e-6)
    hr = h0.astype(np.float64) + _rms(y0)
    assert np.allclose(host(h), hr, rtol=0, atol=1e-6 * np.abs(hr).max() + 1e-7)
    xr = _rms(hr)
    assert np.allclose(host(x[:D]), xr, rtol=0, atol=2e-6 * np.abs(xr).max())
    assert torch.equal(x[D:], torch.full((64,), 7.0, device="cuda"))
    assert torch.equal(y.cpu(), torch.from_numpy(y0))
    # without y: h untouched, x = rms(h)
    h2 = torch.from_numpy(h0.copy()).cuda()
    x2 = torch.empty(D, device="cuda")
    la.residual_norm(h2, x2)
    assert torch.equal(h2.cpu(), torch.from_numpy(h0))
    assert np.allclose(host(x2), _rms(h0), rtol=0, atol=2e-6 * np.abs(_rms(h0)).max())
    # the same call twice gives the same bits
    h3 = torch.from_numpy(h0.copy()).cuda()
    x3 = torch.empty(D, device="cuda")
    la.residual_norm(h3, x3, y)
    assert torch.equal(h3, h) and torch.equal(x3, x[:D])
