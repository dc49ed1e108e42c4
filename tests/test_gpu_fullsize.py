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


def test_gemma_head_b16_one_workspace_calls():
    """rq_logits at B=16 on the full head, three calls on one workspace with other hidden vectors in between:
    nothing a call leaves in the workspace (split vectors, padded codebooks, partial sums, keys) reaches the
    next one (the second call's logits against the oracle; the third, on the first call's vectors,
    bit-identical to the first)."""
    cfg = synth.CONFIGS["gemma_b16"]
    mat, h1, _ = synth.make_head(cfg)
    h2 = synth.gen_hidden(np.random.default_rng(77), cfg.B, mat.D)
    W = to_dev(mat)
    ws = torch.zeros(la.logits_workspace(W, cfg.B, 0), dtype=torch.uint8, device="cuda")
    lg1, am1, _, _ = la.logits(W, dev(h1), softcap=cfg.softcap, ws=ws)
    first = host(lg1).copy()
    lg2, am2, _, _ = la.logits(W, dev(h2), softcap=cfg.softcap, ws=ws)
    _, ref2 = oracle_head(mat, h2, cfg.softcap)
    check_logits(host(lg2), ref2)
    check_argmax(host(am2), host(lg2), ref2)
    lg3, am3, _, _ = la.logits(W, dev(h1), softcap=cfg.softcap, ws=ws)
    assert np.array_equal(host(lg3), first)
    assert np.array_equal(host(am3), host(am1))


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


def test_stress_head_one_call_full():
    """The stress head through rq_logits (matrix cores, one pair per staged slot at K=4096): every logit within
    1e-5 of max|logit| of the oracle (fp32-level, stricter than the bf16-table bound) and the top-50 rules."""
    cfg = synth.CONFIGS["stress"]
    mat, h, _ = synth.make_head(cfg)
    W = to_dev(mat)
    assert la.logits_method(W, cfg.B) == la.RQ_METHOD_MATRIX_CORES
    lg, am, ti, tv = la.logits(W, dev(h), softcap=cfg.softcap, topk=cfg.topk)
    g = host(lg)
    _, ref = oracle_head(mat, h, cfg.softcap)
    worst = check_logits(g, ref)
    tol = 1e-5 * np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
    check_topk(g, host(ti), host(tv), host(am), ref, tol, cfg.topk)
    print(f"stress one call: worst |gpu-oracle|/max|oracle| = {worst:.2e}")


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
        yf = host(la.lut_mlp(Wg, Wu, Wd, xd))   # the fused block
        check_logits(yf, host(y).astype(np.float64))
        og, ou, _, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                                (down.codes, down.codebooks, False), x)
        check_logits(host(g), og)
        check_logits(host(u), ou)
        check_logits(host(y), oy)
        check_logits(yf, oy)
        del Wg, Wu, Wd


@pytest.mark.parametrize("layer", [0, 1, 25])
def test_mlp_layer_packed10_full(layer):
    """The benchmarked 10-bit MLP layer (gate/up/down codes in RQ_CODES_PACKED10, d=2, K=1024, fp32
    codebooks) under the planner's Gemma-shape plans: the fused block and the three matvecs against the
    oracle; a repeated call gives the same bits."""
    x = synth.make_mlp_x()
    xd = dev(x)
    gate, up, down = synth.make_mlp_layer(layer)
    P = [to_dev(m, "packed10") for m in (gate, up, down)]
    y = host(la.lut_mlp(*P, xd))
    g = la.lut_matvec(P[0], xd)
    u = la.lut_matvec(P[1], xd)
    y3 = host(la.lut_matvec(P[2], g, x2=u, prologue=la.RQ_PRO_GELU_TANH_MUL))
    og, ou, _, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                            (down.codes, down.codebooks, False), x)
    check_logits(host(g), og)
    check_logits(host(u), ou)
    check_logits(y3, oy)
    check_logits(y, oy)
    assert np.array_equal(host(la.lut_mlp(*P, xd)), y)   # deterministic


def test_composite_gemma_shapes_teacher_forced():
    """The per-token loop at the Gemma-2-2B shapes (the 256000 x 2304 head, 26 MLP blocks of 9216 x 2304 /
    2304 x 9216) for three tokens, teacher-forced: for every token and block, the block's GPU output against
    the oracle's block on the GPU's input to it; the norms and residual stream against numpy; the next token
    within 2t of the oracle head's maximum on the GPU's final hidden vector."""
    from lut_logits_amd.composite import DecodeLoop
    from test_gpu_composite import check_loop_step
    cfg = synth.CONFIGS["gemma_b1"]
    head, _, _ = synth.make_head(cfg)
    layers = [synth.make_mlp_layer(i) for i in range(synth.MLP_LAYERS)]
    loop = DecodeLoop(to_dev(head), [tuple(to_dev(m) for m in lay) for lay in layers], softcap=cfg.softcap,
                      max_tokens=4, keep_layers=True)
    loop.ids[0] = 1234
    o = O()
    tok = 1234
    for t in range(3):
        loop.step(t)
        nxt = int(loop.ids[t + 1].item())
        ref = check_loop_step(o, head, layers, loop, tok, cfg.softcap)
        tol = 1e-5 * np.abs(ref).max()
        assert ref[0, nxt] >= ref[0].max() - 2 * tol, f"token {t}: {nxt} is not a maximum of the oracle head"
        tok = nxt   # (with a tied head the residual stream keeps the token's own row: often the same token)
