"""CPU oracle for RQ LUT serving -- TEST INFRASTRUCTURE ONLY.

This package is the plain fp64 reference that the HIP path is checked against.
Only the tests, the package smoke check and the bench's CPU-baseline leg may
import it; the library under lut_logits_amd/ never does, and the two share no
code (the seeded input generator is the one module both sides are fed from).

Each function follows the definitions written out at the top of
rq_oracle.c (Gemma-2-2B runtime-compression page, "LUT serving" paragraph
and correctness-check table; Gemma-2-2B MLP RQ page for the MLP matrices).

Arrays are numpy: codebooks fp32 or bf16-as-uint16 [L][M][K][d], codes uint16
[rows][L][M], activations fp32 [B][D].
"""
import ctypes
import os

import numpy as np

from .build import LIB, build as _build_lib

_ERR = {-1: "null pointer", -2: "bad shape", -7: "code >= K"}

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {_ERR.get(rc, 'unknown')}")


class Oracle:
    """ctypes view of one compiled oracle library (the default, or a test build)."""

    def __init__(self, libpath=LIB):
        if libpath == LIB and not os.path.exists(LIB):
            _build_lib()
        self.lib = lib = ctypes.CDLL(libpath)
        i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        lib.oracle_matvec.argtypes = [i64, i32, i32, i32, i32, i32, vp, i32, _u16p, _dp, i32, _dp, i32]
        lib.oracle_logits.argtypes = [i64, i32, i32, i32, i32, i32, vp, i32, _u16p, _fp, i32, dbl, _dp, _dp, i32]
        lib.oracle_build_lut.argtypes = [i32, i32, i32, i32, i32, vp, i32, _dp, i32, _dp]
        lib.oracle_lut_sum.argtypes = [i64, i32, i32, i32, _u16p, _dp, i32, _dp, i32]
        lib.oracle_argmax.argtypes = [_dp, i32, i64, _i32p]
        lib.oracle_argmax.restype = None
        lib.oracle_topk.argtypes = [_dp, i32, i64, i32, _i32p, _dp]
        lib.oracle_decode_rows.argtypes = [i64, i32, i32, i32, i32, i32, vp, i32, _u16p, _i32p, i32, i32, vp, _i64p]
        lib.oracle_softcap.argtypes = [dbl, dbl]
        lib.oracle_softcap.restype = dbl
        lib.oracle_gelu_tanh.argtypes = [dbl]
        lib.oracle_gelu_tanh.restype = dbl
        lib.oracle_gelu_mul.argtypes = [_dp, _dp, i64, _dp]
        lib.oracle_gelu_mul.restype = None
        lib.oracle_check_codes.argtypes = [i64, i32, i32, i32, _u16p]
        lib.oracle_max_threads.argtypes = []

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _mat(codes, cb, cb_bf16):
        codes = np.ascontiguousarray(codes, dtype=np.uint16)
        if codes.ndim != 3 or cb.ndim != 4:
            raise ValueError("codes must be [rows][L][M] and codebooks [L][M][K][d]")
        cb = np.ascontiguousarray(cb, dtype=np.uint16 if cb_bf16 else np.float32)
        rows, L, M = codes.shape
        Lc, Mc, K, d = cb.shape
        if (Lc, Mc) != (L, M):
            raise ValueError("codebook and code shapes disagree")
        return codes, cb, rows, L, M, K, d

    def max_threads(self):
        return self.lib.oracle_max_threads()

    # -- definitions -----------------------------------------------------
    def matvec(self, codes, cb, cb_bf16, x, nthreads=0):
        """y[b][r] = <decoded row r, x[b]> in fp64. x: [B][D] (any float), returns fp64 [B][rows]."""
        codes, cb, rows, L, M, K, d = self._mat(codes, cb, cb_bf16)
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
        B, D = x.shape
        y = np.zeros((B, rows), np.float64)
        _check(self.lib.oracle_matvec(rows, D, M, d, K, L, cb.ctypes.data, int(cb_bf16), _ptr(codes, _u16p),
                                      _ptr(x, _dp), B, _ptr(y, _dp), nthreads or self.max_threads()))
        return y

    def logits(self, codes, cb, cb_bf16, h, softcap, nthreads=0):
        """(z, logits) fp64 [B][V]: decode + matmul, then c*tanh(z/c) (c <= 0: off)."""
        codes, cb, V, L, M, K, d = self._mat(codes, cb, cb_bf16)
        h = np.ascontiguousarray(np.atleast_2d(h), dtype=np.float32)
        B, D = h.shape
        z = np.zeros((B, V), np.float64)
        out = np.zeros((B, V), np.float64)
        _check(self.lib.oracle_logits(V, D, M, d, K, L, cb.ctypes.data, int(cb_bf16), _ptr(codes, _u16p),
                                      _ptr(h, _fp), B, float(softcap), _ptr(z, _dp), _ptr(out, _dp),
                                      nthreads or self.max_threads()))
        return z, out

    def build_lut(self, cb, cb_bf16, x):
        """LUT[b][l][m][k] = <x[b] on subspace m, C[l][m][k]> in fp64, shape [B][L][M][K]."""
        cb = np.ascontiguousarray(cb, dtype=np.uint16 if cb_bf16 else np.float32)
        L, M, K, d = cb.shape
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
        B, D = x.shape
        lut = np.zeros((B, L, M, K), np.float64)
        _check(self.lib.oracle_build_lut(D, M, d, K, L, cb.ctypes.data, int(cb_bf16), _ptr(x, _dp), B, _ptr(lut, _dp)))
        return lut

    def lut_sum(self, codes, lut, nthreads=0):
        """z[b][r] = sum_{l,m} LUT[b][l][m][code[r][l][m]] in fp64."""
        codes = np.ascontiguousarray(codes, dtype=np.uint16)
        lut = np.ascontiguousarray(lut, dtype=np.float64)
        rows, L, M = codes.shape
        B, L2, M2, K = lut.shape
        if (L2, M2) != (L, M):
            raise ValueError("LUT and code shapes disagree")
        z = np.zeros((B, rows), np.float64)
        _check(self.lib.oracle_lut_sum(rows, M, K, L, _ptr(codes, _u16p), _ptr(lut, _dp), B, _ptr(z, _dp),
                                       nthreads or self.max_threads()))
        return z

    def argmax(self, logits):
        logits = np.ascontiguousarray(np.atleast_2d(logits), dtype=np.float64)
        B, V = logits.shape
        out = np.zeros(B, np.int32)
        self.lib.oracle_argmax(_ptr(logits, _dp), B, V, _ptr(out, _i32p))
        return out

    def topk(self, logits, k):
        logits = np.ascontiguousarray(np.atleast_2d(logits), dtype=np.float64)
        B, V = logits.shape
        ids = np.zeros((B, k), np.int32)
        vals = np.zeros((B, k), np.float64)
        _check(self.lib.oracle_topk(_ptr(logits, _dp), B, V, k, _ptr(ids, _i32p), _ptr(vals, _dp)))
        return ids, vals

    def check_codes(self, codes, K):
        """0 when every code of [rows][L][M] is below K, else the oracle's error status."""
        codes = np.ascontiguousarray(codes, dtype=np.uint16)
        rows, L, M = codes.shape
        return self.lib.oracle_check_codes(rows, M, K, L, _ptr(codes, _u16p))

    def decode_rows(self, codes, cb, cb_bf16, ids, out_bf16):
        """Rows [n][D]: fp32 (out_bf16 False) or bf16 bits as uint16; plus the bad-id count."""
        codes, cb, V, L, M, K, d = self._mat(codes, cb, cb_bf16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        n = ids.shape[0]
        D = M * d
        out = np.zeros((n, D), np.uint16 if out_bf16 else np.float32)
        bad = ctypes.c_int64(0)
        _check(self.lib.oracle_decode_rows(V, D, M, d, K, L, cb.ctypes.data, int(cb_bf16), _ptr(codes, _u16p),
                                           _ptr(ids, _i32p), n, int(out_bf16), out.ctypes.data, ctypes.byref(bad)))
        return out, bad.value

    def softcap(self, z, c):
        return np.vectorize(lambda t: self.lib.oracle_softcap(float(t), float(c)), otypes=[np.float64])(z)

    def gelu_tanh(self, t):
        return np.vectorize(lambda v: self.lib.oracle_gelu_tanh(float(v)), otypes=[np.float64])(t)

    def gelu_mul(self, g, u):
        g = np.ascontiguousarray(g, dtype=np.float64)
        u = np.ascontiguousarray(u, dtype=np.float64)
        a = np.zeros_like(g)
        self.lib.oracle_gelu_mul(_ptr(g, _dp), _ptr(u, _dp), g.size, _ptr(a, _dp))
        return a

    def mlp(self, gate, up, down, x, nthreads=0):
        """One MLP block on RQ-coded weights (each a (codes, cb, cb_bf16) triple):
        g = W_gate x, u = W_up x, a = gelu_tanh(g) * u, y = W_down a. Returns (g, u, a, y) in fp64."""
        g = self.matvec(*gate, x, nthreads)
        u = self.matvec(*up, x, nthreads)
        a = self.gelu_mul(g, u)
        y = self.matvec(*down, a, nthreads)
        return g, u, a, y


_default = None


def default():
    """The oracle built from oracle/rq_oracle.c (RQ_ORACLE_LIB names another build of it, such as the
    sanitizer build of the CPU test run)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("RQ_ORACLE_LIB") or LIB)
    return _default
