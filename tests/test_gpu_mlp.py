"""rq_lut_mlp, the fused Gemma-2 MLP block (needs an MI355X).

The block does the arithmetic of the three rq_lut_matvec calls it replaces (gate and up in one launch,
down's activation summed from their partial sums in the finish pass's order); only the number of partial
sums gate and up are split into may differ. So it matches the CPU oracle, matches the three calls to fp32
rounding, is deterministic, and on exact inputs (where no grouping can change a bit) equals them exactly."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
import oracle
from lut_logits_amd import synth
from gpu_util import check_logits, dev, host, to_dev

pytestmark = pytest.mark.gpu

O = oracle.default

SHAPES = [
    # hid, inter, d, K, B
    (96, 160, 2, 64, 1),       # tiny: the planner may use one group for gate/up
    (128, 260, 4, 256, 1),     # d=4, ragged rows
    (64, 200, 1, 128, 1),      # d=1
    (1024, 3000, 2, 256, 1),   # more groups: the finish order with 4 parts per row
    (96, 160, 2, 64, 2),       # two activation vectors: the three-call route
    (128, 256, 8, 256, 1),     # d=8: codewords over two staged words
    (96, 200, 8, 64, 1),       # d=8, ragged rows
]


def _three_calls(Wg, Wu, Wd, xd):
    g = la.lut_matvec(Wg, xd)
    u = la.lut_matvec(Wu, xd)
    return la.lut_matvec(Wd, g, x2=u, prologue=la.RQ_PRO_GELU_TANH_MUL)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["rows", "blocked", "packed10"])
def test_lut_mlp_matches_three_calls_and_oracle(shape, layout):
    hid, inter, d, K, B = shape
    if layout == "rows" and ((2 * hid // d) % 8 or (2 * inter // d) % 8):
        pytest.skip("row-major codes need L*M % 8 == 0")
    rng = np.random.default_rng(hid + inter + d + K + B)
    gate = synth.gen_matrix(rng, inter, hid, hid // d, K, 2, (0.02, 0.005), "f32")
    up = synth.gen_matrix(rng, inter, hid, hid // d, K, 2, (0.02, 0.005), "f32")
    down = synth.gen_matrix(rng, hid, inter, inter // d, K, 2, (0.02, 0.005), "f32")
    x = synth.gen_hidden(rng, B, hid)
    Wg, Wu, Wd = to_dev(gate, layout), to_dev(up, layout), to_dev(down, layout)
    xd = dev(x)
    y = la.lut_mlp(Wg, Wu, Wd, xd)
    y3 = _three_calls(Wg, Wu, Wd, xd)
    check_logits(host(y), host(y3).astype(np.float64))
    assert torch.equal(la.lut_mlp(Wg, Wu, Wd, xd), y)
    _, _, _, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                          (down.codes, down.codebooks, False), x)
    check_logits(host(y), oy)


def test_lut_mlp_gemma_layer_and_reuse():
    """One Gemma-2-2B MLP layer (gate/up 9216x2304, down 2304x9216, d=2, K=1024, L=2, fp32 codebooks):
    close to the oracle and to the three calls; a second call on the same workspace, with another x,
    gives that x's result (nothing carried over)."""
    gate, up, down = synth.make_mlp_layer(0)
    x = synth.make_mlp_x()
    Wg, Wu, Wd = to_dev(gate), to_dev(up), to_dev(down)
    ws = la.workspace(la.lut_mlp_workspace(Wg, Wu, Wd, 1), "cuda")
    xd = dev(x)
    y = la.lut_mlp(Wg, Wu, Wd, xd, ws=ws).clone()
    check_logits(host(y), host(_three_calls(Wg, Wu, Wd, xd)).astype(np.float64))
    _, _, _, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                          (down.codes, down.codebooks, False), x)
    check_logits(host(y), oy)
    x2 = synth.gen_hidden(np.random.default_rng(5), 1, x.shape[1])
    x2d = dev(x2)
    y2 = la.lut_mlp(Wg, Wu, Wd, x2d, ws=ws).clone()
    check_logits(host(y2), host(_three_calls(Wg, Wu, Wd, x2d)).astype(np.float64))
    assert torch.equal(la.lut_mlp(Wg, Wu, Wd, x2d, ws=ws), y2)
    assert not torch.equal(y2, y)


def test_lut_mlp_exact_inputs_gemma_shape():
    """Small-integer codebooks and x at the Gemma MLP shapes: g and u are exact however their partial sums
    are grouped (and equal the oracle's), so the block equals the three calls bit for bit."""
    gate, x = synth.gen_exact(71, 9216, 2304, 1152, 1024, 2, 1)
    up, _ = synth.gen_exact(72, 9216, 2304, 1152, 1024, 2, 1)
    down, _ = synth.gen_exact(73, 2304, 9216, 4608, 1024, 2, 1)
    Wg, Wu, Wd = to_dev(gate), to_dev(up), to_dev(down)
    xd = dev(x)
    g = la.lut_matvec(Wg, xd)
    assert np.array_equal(host(g).astype(np.float64), O().matvec(gate.codes, gate.codebooks, False, x))
    assert torch.equal(la.lut_mlp(Wg, Wu, Wd, xd), _three_calls(Wg, Wu, Wd, xd))


def test_lut_mlp_second_attempt_shapes():
    """The MLP RQ page's second-attempt layer: d=8 throughout, K=1024 for gate/up (10-bit codes), K=256 for
    down (8-bit codes), fp32 codebooks: close to the three matvecs and to the oracle."""
    gate, up, down = synth.make_mlp_v2_layer(0)
    x = synth.make_mlp_x()
    Wg, Wu, Wd = to_dev(gate, "packed10"), to_dev(up, "packed10"), to_dev(down, "packed8")
    xd = dev(x)
    y = la.lut_mlp(Wg, Wu, Wd, xd)
    check_logits(host(y), host(_three_calls(Wg, Wu, Wd, xd)).astype(np.float64))
    og, ou, _, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                            (down.codes, down.codebooks, False), x)
    check_logits(host(la.lut_matvec(Wg, xd)), og)
    check_logits(host(y), oy)
    # the 8-bit stream is half the 16-bit one: 2304 rows x 2304 pairs
    assert Wd.codes.numel() * 2 == 2304 * 2304


def test_lut_mlp_second_attempt_exact_inputs():
    """Exact inputs at the second-attempt shapes (d=8, gate/up K=1024 on 10-bit codes, down K=256 on 8-bit
    codes): gate's fused d=8 build is bit-exact against the oracle, and the block equals the three calls."""
    gate, x = synth.gen_exact(81, 9216, 2304, 288, 1024, 2, 1)
    up, _ = synth.gen_exact(82, 9216, 2304, 288, 1024, 2, 1)
    down, _ = synth.gen_exact(83, 2304, 9216, 1152, 256, 2, 1)
    Wg, Wu, Wd = to_dev(gate, "packed10"), to_dev(up, "packed10"), to_dev(down, "packed8")
    xd = dev(x)
    g = la.lut_matvec(Wg, xd)
    assert np.array_equal(host(g).astype(np.float64), O().matvec(gate.codes, gate.codebooks, False, x))
    assert torch.equal(la.lut_mlp(Wg, Wu, Wd, xd), _three_calls(Wg, Wu, Wd, xd))
