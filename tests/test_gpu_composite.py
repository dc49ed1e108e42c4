"""The per-token decode loop (lut_logits_amd.composite) against the oracle, token by token (needs an MI355X).

The loop feeds each argmax back as the next token on the device. The oracle is run teacher-forced: for
every step it takes the token the GPU chose, rebuilds that token's embedding row, the sqrt(D) scale, the
MLP chain (fp64) and the head, and the GPU's hidden vector and next token must agree with it."""
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
    loop = DecodeLoop(Wh, [tuple(to_dev(m) for m in lay) for lay in layers], softcap=cfg.softcap, max_tokens=8)
    loop.ids[0] = 7
    o = O()
    scale = np.float32(np.sqrt(cfg.D))
    tokens = [7]
    for t in range(8):
        x_gpu = host(loop.step(t))
        nxt = int(loop.ids[t + 1].item())
        # oracle, teacher-forced on the GPU's token t
        row, _ = o.decode_rows(head.codes, head.codebooks, head.cb_is_bf16, np.array([tokens[-1]], np.int32), False)
        y = row.astype(np.float32) * scale              # the loop's fp32 scaling of the fp32 row
        for gate, up, down in layers:
            _, _, _, y = o.mlp(*((m.codes, m.codebooks, False) for m in (gate, up, down)), y)
        check_logits(x_gpu, y)
        _, ref = o.logits(head.codes, head.codebooks, head.cb_is_bf16, x_gpu, cfg.softcap)
        tol = 1e-5 * np.abs(ref).max()
        assert ref[0, nxt] >= ref[0].max() - 2 * tol, f"step {t}: token {nxt} is not a maximum of the oracle"
        tokens.append(nxt)
    assert torch.equal(loop.ids[:9].cpu(), torch.tensor(tokens, dtype=torch.int32))
    # a second run from the same token repeats the sequence (deterministic)
    ids2 = loop.run(7, 8).clone()
    assert torch.equal(ids2.cpu(), torch.tensor(tokens, dtype=torch.int32))
