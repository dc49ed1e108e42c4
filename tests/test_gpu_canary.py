"""Workspace guards: every entry point that takes a workspace is handed exactly the size its query returns,
cut out of a larger buffer whose bytes are all 0xFF (a NaN pattern as fp32 and bf16, key 0xFF.. as an
integer). After the call the 256 bytes before the workspace and the 4 KiB after it must still hold 0xFF,
and the outputs must be bit-identical to those of a call on a zeroed workspace of generous size: the
kernels write nothing outside their workspace and read nothing of it they did not write first."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
from lut_logits_amd import synth
from gpu_util import dev, host, to_dev

pytestmark = pytest.mark.gpu

HEAD, TAIL = 256, 4096


def guarded(need):
    """(buffer, workspace view of exactly `need` bytes at offset HEAD), all bytes 0xFF."""
    buf = torch.full((HEAD + need + TAIL,), 0xFF, dtype=torch.uint8, device="cuda")
    return buf, buf[HEAD:HEAD + need]


def roomy(need):
    return torch.zeros(need + (1 << 20), dtype=torch.uint8, device="cuda")


def check_guards(buf, need):
    b = host(buf)
    assert np.all(b[:HEAD] == 0xFF), "bytes before the workspace were written"
    tail = b[HEAD + need:]
    bad = np.nonzero(tail != 0xFF)[0]
    assert bad.size == 0, f"{bad.size} bytes after the workspace were written, first at +{bad[0] if bad.size else 0}"


def same(a, b):
    for x, y in zip(a, b):
        if x is None or y is None:
            assert x is None and y is None
            continue
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)


def _mat(seed, rows, D, M, K, L, cb_dtype="f32"):
    rng = np.random.default_rng(seed)
    sig = tuple(0.02 * 0.25 ** l for l in range(L))
    return synth.gen_matrix(rng, rows, D, M, K, L, sig, cb_dtype), rng


@pytest.mark.parametrize("B,topk,lut_dtype", [(1, 0, "f32"), (20, 5, "bf16"), (3, 0, "f32")])
def test_lut_logits_workspace_guard(B, topk, lut_dtype):
    mat, rng = _mat(300 + B, 9000, 96, 16, 256, 2)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(synth.gen_hidden(rng, B, 96)), lut_dtype=lut_dtype)
    need = la.lut_logits_workspace(W, B, topk, lut_dtype)
    buf, ws = guarded(need)
    got = la.lut_logits(W, lut, B, topk=topk, ws=ws)
    want = la.lut_logits(W, lut, B, topk=topk, ws=roomy(need))
    torch.cuda.synchronize()
    check_guards(buf, need)
    same(got, want)
    assert torch.isfinite(got[0]).all()


@pytest.mark.parametrize("B,K,cb_dtype", [(16, 256, "bf16"), (64, 2048, "bf16"), (1, 256, "f32"), (16, 256, "f32")])
def test_logits_workspace_guard(B, K, cb_dtype):
    """rq_logits on the matrix cores (bf16 codebooks, B >= 16: K <= 1024, and one pair per staged slot above it)
    and on the table path (fp32 codebooks)."""
    mat, rng = _mat(320 + B, 3000, 96, 16, K, 2, cb_dtype)
    W = to_dev(mat)
    h = dev(synth.gen_hidden(rng, B, 96))
    need = la.logits_workspace(W, B, 4)
    buf, ws = guarded(need)
    got = la.logits(W, h, topk=4, ws=ws)
    want = la.logits(W, h, topk=4, ws=roomy(need))
    torch.cuda.synchronize()
    check_guards(buf, need)
    same(got, want)
    want_method = la.RQ_METHOD_MATRIX_CORES if B >= 16 and cb_dtype == "bf16" else la.RQ_METHOD_TABLE
    assert la.logits_method(W, B) == want_method


def test_matvec_and_mlp_workspace_guard():
    rng = np.random.default_rng(340)
    gate, up = (synth.gen_matrix(rng, 160, 96, 48, 64, 2, (0.02, 0.005), "f32") for _ in range(2))
    down = synth.gen_matrix(rng, 96, 160, 80, 64, 2, (0.02, 0.005), "f32")
    Wg, Wu, Wd = (la.to_device(m) for m in (gate, up, down))
    x = dev(synth.gen_hidden(rng, 1, 96))
    need = la.lut_matvec_workspace(Wg, 1)
    buf, ws = guarded(need)
    got = la.lut_matvec(Wg, x, ws=ws)
    want = la.lut_matvec(Wg, x, ws=roomy(need))
    need2 = la.lut_mlp_workspace(Wg, Wu, Wd, 1)
    buf2, ws2 = guarded(need2)
    got2 = la.lut_mlp(Wg, Wu, Wd, x, ws=ws2)
    want2 = la.lut_mlp(Wg, Wu, Wd, x, ws=roomy(need2))
    torch.cuda.synchronize()
    check_guards(buf, need)
    check_guards(buf2, need2)
    assert torch.equal(got, want) and torch.equal(got2, want2)


@pytest.mark.parametrize("B", [1, 40])
def test_dense_workspace_guard(B):
    mat, rng = _mat(360 + B, 3000, 96, 16, 256, 2, "bf16")
    W = to_dev(mat)
    E = la.pack_dense(la.decode_rows(W, torch.arange(3000, dtype=torch.int32, device="cuda"), "bf16"))
    h = dev(synth.gen_hidden(rng, B, 96))
    need = la.dense_logits_workspace(3000, B)
    buf, ws = guarded(need)
    got = la.dense_logits(E, h, ws=ws)
    want = la.dense_logits(E, h, ws=roomy(need))
    torch.cuda.synchronize()
    check_guards(buf, need)
    same(got, want)
