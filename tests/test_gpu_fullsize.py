"""HIP path vs the CPU oracle at the full workload sizes, in the configuration the benchmark times
(blocked code layout, the planner's own tiling, the same seeds). Every output is compared: the
oracle's fp64 decode+matmul finishes the whole 256000-row head in seconds on the host's cores."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
import oracle
from lut_logits_amd import synth
from gpu_util import bf16_table_tol, check_argmax, check_logits, check_topk, dev, host, oracle_head, to_dev

# the oracle's full-size passes take seconds to tens of seconds on the host
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

O = oracle.default


@pytest.mark.parametrize("layout", ["blocked", "packed10"])
def test_gemma_head_b1_full(layout):
    """Gemma-2-2B head at decode: 256000 logits + argmax, and the 64 input rows decoded to bf16, from the
    16-bit blocked codes and from the 10-bit code stream."""
    cfg = synth.CONFIGS["gemma_b1"]
    mat, h, ids = synth.make_head(cfg)
    W = to_dev(mat, layout)
    rows = la.decode_rows(W, dev(ids), "bf16")
    assert np.array_equal(host(rows).view(np.uint16),
                          O().decode_rows(mat.codes, mat.codebooks, True, ids, True)[0])
    lut = la.build_lut(W, dev(h))
    lg, am, _, _ = la.lut_logits(W, lut, 1, softcap=cfg.softcap)
    _, ref = oracle_head(mat, h, cfg.softcap)
    worst = check_logits(host(lg), ref)
    check_argmax(host(am), host(lg), ref)
    print(f"gemma B=1 {layout}: worst |gpu-oracle|/max|oracle| = {worst:.2e}")


@pytest.mark.parametrize("name", ["gemma_b16", "gemma_b128"])
def test_gemma_head_batched_full(name):
    """The same head with B=16 and B=128 hidden vectors: [B][256000] logits and per-vector argmax."""
    cfg = synth.CONFIGS[name]
    mat, h, _ = synth.make_head(cfg)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h))
    lg, am, _, _ = la.lut_logits(W, lut, cfg.B, softcap=cfg.softcap)
    _, ref = oracle_head(mat, h, cfg.softcap)
    worst = check_logits(host(lg), ref)
    check_argmax(host(am), host(lg), ref)
    print(f"{name}: worst |gpu-oracle|/max|oracle| = {worst:.2e}")


@pytest.mark.parametrize("name,layout", [("gemma_b16", "blocked"), ("gemma_b128", "blocked"),
                                         ("gemma_b16", "packed10")])
def test_gemma_head_one_call_full(name, layout):
    """rq_logits on the full head at B=16 and B=128 (the matrix-core method): every logit and argmax."""
    cfg = synth.CONFIGS[name]
    mat, h, _ = synth.make_head(cfg)
    W = to_dev(mat, layout)
    assert la.logits_method(W, cfg.B) == la.RQ_METHOD_MATRIX_CORES
    lg, am, _, _ = la.logits(W, dev(h), softcap=cfg.softcap)
    _, ref = oracle_head(mat, h, cfg.softcap)
    worst = check_logits(host(lg), ref)
    check_argmax(host(am), host(lg), ref)
    print(f"{name} {layout} one call: worst |gpu-oracle|/max|oracle| = {worst:.2e}")


def test_stress_head_full():
    """Stress head: K=4096, L=4, B=64, bf16 table, softcap 30 and per-vector top-50."""
    cfg = synth.CONFIGS["stress"]
    mat, h, _ = synth.make_head(cfg)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h), lut_dtype="bf16")
    lg, am, ti, tv = la.lut_logits(W, lut, cfg.B, softcap=cfg.softcap, lut_dtype="bf16", topk=cfg.topk)
    g = host(lg)
    del lut
    _, ref = oracle_head(mat, h, cfg.softcap)
    tolv = bf16_table_tol(mat, h, ref)
    for b in range(cfg.B):
        err = np.abs(g[b].astype(np.float64) - ref[b])
        assert np.all(err <= tolv[b]), f"b={b}: {int((err > tolv[b]).sum())} logits beyond the bf16-table bound"
    check_topk(g, host(ti), host(tv), host(am), ref, tolv, cfg.topk)


def test_mlp_26_layers_full():
    """All 26 Gemma-2-2B MLP layers (independent codes and codebooks, the same x): g, u and y of every layer,
    and rq_lut_mlp's y against the three calls."""
    x = synth.make_mlp_x()
    xd = dev(x)
    for i in range(synth.MLP_LAYERS):
        gate, up, down = synth.make_mlp_layer(i)
        Wg, Wu, Wd = to_dev(gate), to_dev(up), to_dev(down)
        g = la.lut_matvec(Wg, xd)
        u = la.lut_matvec(Wu, xd)
        y = la.lut_matvec(Wd, g, x2=u, prologue=la.RQ_PRO_GELU_TANH_MUL)
        check_logits(host(la.lut_mlp(Wg, Wu, Wd, xd)), host(y).astype(np.float64))   # the fused block
        og, ou, _, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                                (down.codes, down.codebooks, False), x)
        check_logits(host(g), og)
        check_logits(host(u), ou)
        check_logits(host(y), oy)
        del Wg, Wu, Wd
