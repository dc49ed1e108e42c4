"""The Python binding refuses tensors of the wrong dtype, shape, layout or device before any pointer
reaches the library (no GPU needed: every call here fails in the binding's own checks).

The C ABI sees only pointers and sizes, so a float64 activation, an int64 id vector, a bf16 table
passed as fp32 or a short output buffer would otherwise be read or written past its end."""
import pytest
import torch

import lut_logits_amd as la
from lut_logits_amd import binding as B


def _matrix(rows=64, D=12, M=4, K=8, L=2, cb_dtype="f32"):
    d = D // M
    cb = torch.zeros((L, M, K, d), dtype=torch.float32 if cb_dtype == "f32" else torch.int16)
    codes = torch.zeros(B.blocked_codes_bytes(rows, L, M) // 2, dtype=torch.int16)
    return B.DeviceMatrix(rows, D, M, K, L, cb_dtype, cb, codes, "blocked")


W = _matrix()


def _raises(fn, what):
    with pytest.raises((ValueError, TypeError)) as e:
        fn()
    assert what in str(e.value), str(e.value)


def test_build_lut_checks():
    _raises(lambda: la.build_lut(W, torch.zeros((1, 12), dtype=torch.float64)), "dtype")
    _raises(lambda: la.build_lut(W, torch.zeros((1, 11))), "shape")
    _raises(lambda: la.build_lut(W, torch.zeros(12)), "shape")
    _raises(lambda: la.build_lut(W, torch.zeros((12, 2)).t()), "contiguous")
    _raises(lambda: la.build_lut(W, torch.zeros((2, 24))[:, :12]), "contiguous")
    _raises(lambda: la.build_lut(W, torch.zeros((1, 12))), "GPU")   # every other check passed
    _raises(lambda: la.build_lut(W, torch.zeros((2, 12)), x2=torch.zeros((1, 12)),
                                 prologue=la.RQ_PRO_GELU_TANH_MUL), "shape")
    n = B.lut_bytes(W, 1, "f32") // 4
    _raises(lambda: la.build_lut(W, torch.zeros((1, 12)), out=torch.zeros(n - 1)), "elements")
    _raises(lambda: la.build_lut(W, torch.zeros((1, 12)), lut_dtype="bf16", out=torch.zeros(n)), "dtype")


def test_lut_logits_table_dtype_from_tensor():
    n = B.lut_bytes(W, 1, "f32") // 4
    # an int16 tensor holds bf16 entries: asking for fp32 reads would read twice its bytes
    _raises(lambda: la.lut_logits(W, torch.zeros(n, dtype=torch.int16), 1, lut_dtype="f32"), "lut_dtype")
    _raises(lambda: la.lut_logits(W, torch.zeros(n, dtype=torch.float64), 1), "dtype")
    _raises(lambda: la.lut_logits(W, torch.zeros(n - 4), 1), "elements")
    _raises(lambda: la.lut_logits(W, torch.zeros(n * 2), 1), "elements")   # the table of B=2, called with B=1
    assert B._lut_dtype_of(torch.zeros(4, dtype=torch.int16), None) == "bf16"
    assert B._lut_dtype_of(torch.zeros(4), None) == "f32"


def test_head_outputs_checked():
    n = B.lut_bytes(W, 2, "f32") // 4
    lut = torch.zeros(n)
    _raises(lambda: la.lut_logits(W, lut, 2, out=torch.zeros((1, 64))), "elements")
    _raises(lambda: la.lut_logits(W, lut, 2, out=torch.zeros((2, 64), dtype=torch.float16)), "dtype")
    _raises(lambda: la.lut_logits(W, lut, 2, argmax_out=torch.zeros(2, dtype=torch.int64)), "dtype")
    _raises(lambda: la.lut_logits(W, lut, 2, argmax_out=torch.zeros(1, dtype=torch.int32)), "elements")
    _raises(lambda: la.logits(W, torch.zeros((2, 11))), "shape")
    _raises(lambda: la.logits(W, torch.zeros((2, 12), dtype=torch.bfloat16)), "dtype")


def test_decode_rows_checks():
    _raises(lambda: la.decode_rows(W, torch.zeros(4, dtype=torch.int64)), "dtype")   # torch's default integer
    _raises(lambda: la.decode_rows(W, torch.zeros((2, 2), dtype=torch.int32)), "shape")
    _raises(lambda: la.decode_rows(W, torch.zeros(4, dtype=torch.int32), out=torch.zeros((4, 11))), "elements")
    _raises(lambda: la.decode_rows(W, torch.zeros(4, dtype=torch.int32), "bf16", out=torch.zeros((4, 12))), "dtype")
    _raises(lambda: la.decode_rows(W, torch.zeros(4, dtype=torch.int32), bad_ids=torch.zeros(1)), "dtype")


def test_matvec_and_mlp_checks():
    _raises(lambda: la.lut_matvec(W, torch.zeros((1, 13))), "shape")
    _raises(lambda: la.lut_matvec(W, torch.zeros((1, 12)), x2=torch.zeros((1, 12), dtype=torch.float64)), "dtype")
    _raises(lambda: la.lut_matvec(W, torch.zeros((1, 12)), out=torch.zeros((1, 63))), "elements")
    up = _matrix()
    down = _matrix(rows=12, D=64, M=32)
    _raises(lambda: la.lut_mlp(W, up, down, torch.zeros((1, 64))), "shape")
    _raises(lambda: la.lut_mlp(W, up, down, torch.zeros((1, 12)), out=torch.zeros((1, 64))), "elements")


def test_workspace_and_dense_checks():
    lut = torch.zeros(B.lut_bytes(W, 1, "f32") // 4)
    _raises(lambda: la.lut_logits(W, lut, 1, ws=torch.zeros(4096, dtype=torch.float32)), "dtype")
    _raises(lambda: la.pack_dense(torch.zeros((64, 16), dtype=torch.float32)), "dtype")
    _raises(lambda: la.residual_norm(torch.zeros(16), torch.zeros(8)), "elements")
    _raises(lambda: la.residual_norm(torch.zeros(16, dtype=torch.float64), torch.zeros(16)), "dtype")
    _raises(lambda: la.residual_norm(torch.zeros(16), torch.zeros(16), torch.zeros(15)), "elements")
    _raises(lambda: la.residual_norm(torch.zeros(16), torch.zeros(16)), "GPU")
    _raises(lambda: la.dense_logits(torch.zeros((64, 16), dtype=torch.int16), torch.zeros((1, 16))), "DenseHead")
    head = la.DenseHead(torch.zeros(la.dense_tiled_bytes(64, 16) // 2, dtype=torch.int16), 64, 16)
    assert head.nbytes == 4 * 1 * 1024
    _raises(lambda: la.dense_logits(head, torch.zeros((1, 8))), "shape")
    short = la.DenseHead(torch.zeros(100, dtype=torch.int16), 64, 16)
    _raises(lambda: la.dense_logits(short, torch.zeros((1, 16))), "elements")
