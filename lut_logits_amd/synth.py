"""Seeded synthetic inputs for RQ-coded matrices.

This module is the only code that both the HIP path and the CPU oracle are fed
from. It draws random numbers and stores them in the formats the library
reads; it holds none of the method's arithmetic (no decode, no table, no
softcap).

Shapes and value distributions follow the pages' workloads:
  - the Gemma-2-2B tied embedding / head, 256,000 x 2,304 coded with M=384
    subspaces of d=6, K=1,024 codewords and L=2 residual levels
    (runtime-compression page, "LUT serving" paragraph; combined RQ+NF4 page,
    embedding paragraph);
  - the Gemma-2-2B MLP matrices, gate/up 9,216 x 2,304 and down 2,304 x 9,216,
    each with its own codebooks (MLP RQ page, compression paragraph).
No trained codebooks exist here, so codewords are Gaussian with per-level
scales, codes are uniform over [0, K) and hidden vectors are N(0, 1).

Generator: numpy PCG64 via default_rng(seed). Draw order within one seed:
codebooks level by level, then codes, then hidden vectors, then token ids.
"""
from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Storage conversion for inputs only (finite values)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class RQMatrix:
    """Host copy of one RQ-coded matrix W[rows][D] (D = M*d).

    codes: uint16 [rows][L][M];  codebooks: fp32 [L][M][K][d], or the bf16 bit
    patterns as uint16 when cb_dtype == "bf16"."""
    rows: int
    D: int
    M: int
    d: int
    K: int
    L: int
    cb_dtype: str
    codebooks: np.ndarray
    codes: np.ndarray

    @property
    def cb_is_bf16(self):
        return self.cb_dtype == "bf16"

    def codebooks_f32(self):
        return bf16_bits_to_f32(self.codebooks) if self.cb_is_bf16 else self.codebooks


@dataclass
class Config:
    name: str
    V: int            # rows of the coded matrix (vocabulary, or out_features)
    D: int
    M: int
    K: int
    L: int
    sigmas: tuple     # per-level std of the codewords
    cb_dtype: str
    B: int
    seed: int
    softcap: float = 30.0
    n_ids: int = 0
    topk: int = 0
    lut_dtype: str = "f32"
    extra: dict = field(default_factory=dict)

    @property
    def d(self):
        return self.D // self.M


# The workloads the tests and the bench run.
CONFIGS = {
    "tiny": Config("tiny", V=4096, D=96, M=16, K=256, L=2, sigmas=(0.02, 0.005), cb_dtype="f32",
                   B=1, seed=1, n_ids=8),
    "gemma_b1": Config("gemma_b1", V=256000, D=2304, M=384, K=1024, L=2, sigmas=(0.02, 0.005),
                       cb_dtype="bf16", B=1, seed=2, n_ids=64),
    "gemma_b16": Config("gemma_b16", V=256000, D=2304, M=384, K=1024, L=2, sigmas=(0.02, 0.005),
                        cb_dtype="bf16", B=16, seed=3),
    "gemma_b128": Config("gemma_b128", V=256000, D=2304, M=384, K=1024, L=2, sigmas=(0.02, 0.005),
                         cb_dtype="bf16", B=128, seed=3),
    "stress": Config("stress", V=256000, D=2304, M=384, K=4096, L=4, sigmas=(0.02, 0.008, 0.003, 0.001),
                     cb_dtype="bf16", B=64, seed=5, topk=50, lut_dtype="bf16"),
}

# Gemma-2-2B MLP shapes: gate/up W[9216][2304] and down W[2304][9216], rows coded over the
# input dimension with d=2, K=1024, L=2, fp32 codebooks per matrix; layer i uses seed 4000+i.
MLP_LAYERS = 26
MLP_HIDDEN = 2304
MLP_INTER = 9216
MLP_D_SUB = 2
MLP_K = 1024
MLP_L = 2
MLP_SIGMAS = (0.02, 0.005)
MLP_X_SEED = 4


def gen_matrix(rng, rows, D, M, K, L, sigmas, cb_dtype):
    """Draw codebooks [L][M][K][d] (level l ~ N(0, sigmas[l])) then uniform codes [rows][L][M]."""
    if D % M:
        raise ValueError("D must be a multiple of M")
    d = D // M
    cb = np.empty((L, M, K, d), np.float32)
    for l in range(L):
        cb[l] = rng.normal(0.0, sigmas[l], size=(M, K, d)).astype(np.float32)
    codes = rng.integers(0, K, size=(rows, L, M), dtype=np.uint16)
    store = f32_to_bf16_bits(cb) if cb_dtype == "bf16" else cb
    return RQMatrix(rows, D, M, d, K, L, cb_dtype, store, codes)


def gen_hidden(rng, B, D):
    return rng.standard_normal((B, D), dtype=np.float32)


def gen_ids(rng, n, V):
    return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def make_head(cfg, B=None, V=None):
    """(matrix, h [B][D] fp32, ids [n_ids] int32) for a head config; V may be cut for sampling."""
    rng = np.random.default_rng(cfg.seed)
    rows = cfg.V if V is None else V
    mat = gen_matrix(rng, rows, cfg.D, cfg.M, cfg.K, cfg.L, cfg.sigmas, cfg.cb_dtype)
    h = gen_hidden(rng, cfg.B if B is None else B, cfg.D)
    ids = gen_ids(rng, cfg.n_ids, rows)
    return mat, h, ids


def make_mlp_layer(i, inter=MLP_INTER, hidden=MLP_HIDDEN):
    """(gate, up, down) RQ matrices of layer i (seed 4000+i)."""
    rng = np.random.default_rng(4000 + i)
    m_in = hidden // MLP_D_SUB
    m_mid = inter // MLP_D_SUB
    gate = gen_matrix(rng, inter, hidden, m_in, MLP_K, MLP_L, MLP_SIGMAS, "f32")
    up = gen_matrix(rng, inter, hidden, m_in, MLP_K, MLP_L, MLP_SIGMAS, "f32")
    down = gen_matrix(rng, hidden, inter, m_mid, MLP_K, MLP_L, MLP_SIGMAS, "f32")
    return gate, up, down


# The MLP RQ page's second attempt: subspaces of 8 values, K chosen per matrix (1024 for gate/up,
# 256 for down, whose codes fit 8 bits), fp32 codebooks, two levels.
MLP_V2_D_SUB = 8
MLP_V2_K_GATE_UP = 1024
MLP_V2_K_DOWN = 256


def make_mlp_v2_layer(i, inter=MLP_INTER, hidden=MLP_HIDDEN):
    """(gate, up, down) RQ matrices of layer i in the second-attempt shapes (seed 5000+i)."""
    rng = np.random.default_rng(5000 + i)
    m_in = hidden // MLP_V2_D_SUB
    m_mid = inter // MLP_V2_D_SUB
    gate = gen_matrix(rng, inter, hidden, m_in, MLP_V2_K_GATE_UP, MLP_L, MLP_SIGMAS, "f32")
    up = gen_matrix(rng, inter, hidden, m_in, MLP_V2_K_GATE_UP, MLP_L, MLP_SIGMAS, "f32")
    down = gen_matrix(rng, hidden, inter, m_mid, MLP_V2_K_DOWN, MLP_L, MLP_SIGMAS, "f32")
    return gate, up, down


def make_mlp_x(B=1, hidden=MLP_HIDDEN):
    return gen_hidden(np.random.default_rng(MLP_X_SEED), B, hidden)


def gen_exact(seed, rows, D, M, K, L, B, cb_dtype="f32", cmax=8, hmax=4):
    """Inputs on which every fp32 product and partial sum is exact.

    Codewords are integers in [-cmax, cmax] times 2^-6 and hidden values are
    integers in [-hmax, hmax]; any sum of at most D*L products stays a multiple
    of 2^-6 far below 2^18, so no rounding happens in fp32 or bf16 storage."""
    rng = np.random.default_rng(seed)
    d = D // M
    cb = (rng.integers(-cmax, cmax + 1, size=(L, M, K, d)).astype(np.float32) * np.float32(2.0 ** -6))
    codes = rng.integers(0, K, size=(rows, L, M), dtype=np.uint16)
    h = rng.integers(-hmax, hmax + 1, size=(B, D)).astype(np.float32)
    store = f32_to_bf16_bits(cb) if cb_dtype == "bf16" else cb
    return RQMatrix(rows, D, M, d, K, L, cb_dtype, store, codes), h
