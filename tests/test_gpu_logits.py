"""rq_logits, the one-call head, on both of its methods (needs an MI355X).

The matrix-core method stages bf16 codebooks on chip and contracts them with the hidden vectors split
into three bf16 parts; the table method builds the fp32 table and runs the lookup+sum. Both are compared
with the CPU oracle through the C ABI."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
import oracle
from lut_logits_amd import synth
from gpu_util import check_argmax, check_logits, check_topk, dev, host, oracle_head, to_dev

pytestmark = pytest.mark.gpu

O = oracle.default

MM_EXACT = [
    # rows, D, M, K, L, B
    (4097, 96, 16, 256, 2, 16),     # d=6, one column tile, ragged rows
    (2049, 96, 16, 1024, 2, 8),     # the smallest batch routed to the matrix cores, K at its maximum
    (3000, 102, 17, 1000, 2, 33),   # odd M: the last code block is partly empty; K not a power of two; 33 of 64 columns
    (1500, 96, 48, 64, 2, 20),      # d=2
    (1200, 96, 24, 128, 3, 64),     # d=4, L=3, four column tiles
    (700, 64, 8, 256, 1, 100),      # d=8, one code block; blocked: all 100 in one workgroup, packed10: 64 + 36
    (1, 6, 1, 1, 1, 16),            # one row, one codeword, one pair
    # up to 16 vectors on blocked codes: half-blocks of the padded codebook copy loaded into LDS
    (3000, 102, 17, 1000, 2, 16),   # odd M, K not a power of two
    (1500, 96, 48, 64, 2, 12),      # d=2
    (1200, 96, 24, 128, 3, 16),     # d=4, L=3
    (700, 64, 8, 256, 1, 9),        # d=8, one code block
    (2100, 96, 16, 1023, 2, 16),    # K*d not whole 16-byte words
    # 65..128 vectors on blocked codes: eight column tiles in one workgroup, half-blocks loaded into LDS
    (4097, 96, 16, 1024, 2, 128),   # d=6 at the largest K, ragged rows
    (3000, 102, 17, 1000, 2, 65),   # odd M (the last block partly empty), K not a power of two, 65 of 128
    (1500, 96, 48, 64, 2, 128),     # d=2
    (1200, 96, 24, 128, 3, 96),     # d=4, L=3
    (3, 6, 1, 2, 1, 128),           # three rows, one pair
]


@pytest.mark.parametrize("shape", MM_EXACT, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["blocked", "packed10"])
def test_logits_matrix_cores_exact(shape, layout):
    """Small-integer inputs: every product and sum is exact in fp32, so z matches the oracle bit for bit
    (16-bit blocked codes: two sub-blocks per code block; 10-bit codes: three)."""
    rows, D, M, K, L, B = shape
    mat, h = synth.gen_exact(rows + 7 * K, rows, D, M, K, L, B, cb_dtype="bf16")
    W = to_dev(mat, layout)
    assert la.logits_method(W, B) == la.RQ_METHOD_MATRIX_CORES
    lg, am, _, _ = la.logits(W, dev(h), softcap=0.0)
    z, _ = O().logits(mat.codes, mat.codebooks, True, h, 0.0)
    got = host(lg)
    assert np.array_equal(got.astype(np.float64), z)
    assert np.array_equal(host(am), np.argmax(got, axis=1).astype(np.int32))


MM_ONE_PAIR_EXACT = [
    # rows, D, M, K, L, B: K above 1024, one (level, subspace) pair per staged slot
    (3000, 96, 16, 2048, 2, 16),    # d=6, one column tile
    (2500, 96, 16, 4096, 4, 64),    # the stress head's K and L, four column tiles
    (1000, 96, 48, 1500, 2, 33),    # d=2, K not a power of two, 33 of 64 columns
    (700, 64, 8, 3000, 1, 100),     # d=8, one code block, two batch tiles
    (4097, 102, 17, 1028, 3, 8),    # odd M (last block partly empty), K just above 1024, ragged rows
]


@pytest.mark.parametrize("shape", MM_ONE_PAIR_EXACT, ids=lambda s: "x".join(map(str, s)))
def test_logits_matrix_cores_one_pair_exact(shape):
    """K above 1024 (blocked codes): one pair per staged slot, copied straight into LDS, the three bf16 parts of
    h in the MFMA's k-slots. Small-integer inputs make every product and sum exact, so z matches the oracle bit
    for bit."""
    rows, D, M, K, L, B = shape
    mat, h = synth.gen_exact(rows + 3 * K, rows, D, M, K, L, B, cb_dtype="bf16")
    W = to_dev(mat)
    assert la.logits_method(W, B) == la.RQ_METHOD_MATRIX_CORES
    lg, am, _, _ = la.logits(W, dev(h), softcap=0.0)
    z, _ = O().logits(mat.codes, mat.codebooks, True, h, 0.0)
    got = host(lg)
    assert np.array_equal(got.astype(np.float64), z)
    assert np.array_equal(host(am), np.argmax(got, axis=1).astype(np.int32))


def test_logits_one_pair_float_parity():
    """Gaussian inputs at K=4096, L=4 (the stress head's codebooks, 4000 rows, B=64): within 1e-5 of max|logit|
    of the oracle, softcap and top-10 included."""
    cfg = synth.CONFIGS["stress"]
    mat, h, _ = synth.make_head(cfg, V=4000)
    W = to_dev(mat)
    assert la.logits_method(W, cfg.B) == la.RQ_METHOD_MATRIX_CORES
    lg, am, ti, tv = la.logits(W, dev(h), softcap=cfg.softcap, topk=10)
    _, ref = oracle_head(mat, h, cfg.softcap)
    g = host(lg)
    check_logits(g, ref)
    tol = 1e-5 * np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
    check_topk(g, host(ti), host(tv), host(am), ref, tol, 10)


def test_logits_split_reaches_fp32():
    """One subspace of d=6, L=1: z is a 6-term dot product. Splitting h into three bf16 parts keeps it to
    fp32 rounding (|err| <= 2^-20 |z|-scale); two parts would leave ~2^-16 and fail this bound."""
    rng = np.random.default_rng(7)
    mat = synth.gen_matrix(rng, 64, 6, 1, 16, 1, (1.0,), "bf16")
    h = synth.gen_hidden(rng, 16, 6)
    W = to_dev(mat)
    assert la.logits_method(W, 16) == la.RQ_METHOD_MATRIX_CORES
    lg, _, _, _ = la.logits(W, dev(h), softcap=0.0)
    z, _ = O().logits(mat.codes, mat.codebooks, True, h, 0.0)
    c = synth.bf16_bits_to_f32(mat.codebooks).astype(np.float64)[0, 0]          # [K][6]
    scale = np.abs(h.astype(np.float64)) @ np.abs(c[mat.codes[:, 0, 0]]).T     # sum_j |h_j c_j|
    assert np.all(np.abs(host(lg) - z) <= 2.0 ** -20 * scale)


@pytest.mark.parametrize("B", [3, 8, 16, 24, 48, 128])
def test_logits_float_parity(B):
    """Gaussian inputs at the Gemma subspace shape (d=6, K=1024, L=2, bf16 codebooks), softcap 30, argmax."""
    rng = np.random.default_rng(300 + B)
    mat = synth.gen_matrix(rng, 5000, 96, 16, 1024, 2, (0.02, 0.005), "bf16")
    h = synth.gen_hidden(rng, B, 96)
    W = to_dev(mat)
    want = la.RQ_METHOD_MATRIX_CORES if B >= 8 else la.RQ_METHOD_TABLE
    assert la.logits_method(W, B) == want
    lg, am, _, _ = la.logits(W, dev(h), softcap=30.0)
    _, ref = oracle_head(mat, h, 30.0)
    check_logits(host(lg), ref)
    check_argmax(host(am), host(lg), ref)


def test_logits_topk_and_outputs():
    """Top-k on the matrix-core method; argmax alone without a logits output; canaries past [B][rows];
    repeated calls give identical bits."""
    rng = np.random.default_rng(400)
    mat = synth.gen_matrix(rng, 3001, 96, 16, 512, 2, (0.02, 0.005), "bf16")
    h = synth.gen_hidden(rng, 20, 96)
    W, hd = to_dev(mat), dev(h)
    buf = torch.full((20 * 3001 + 64,), float("nan"), device="cuda")
    lg, am, ti, tv = la.logits(W, hd, softcap=30.0, topk=10, out=buf[:20 * 3001].view(20, 3001))
    assert np.all(np.isnan(host(buf[20 * 3001:])))
    g = host(lg)
    _, ref = oracle_head(mat, h, 30.0)
    check_logits(g, ref)
    tol = 1e-5 * np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
    check_topk(g, host(ti), host(tv), host(am), ref, tol, 10)
    lg2, am2, _, _ = la.logits(W, hd, softcap=30.0)
    _, am3, _, _ = la.logits(W, hd, softcap=30.0, logits=False)
    assert torch.equal(lg, lg2) and torch.equal(am, am2) and torch.equal(am, am3)


def test_logits_table_method_matches_two_call_form():
    """Below the matrix-core batch (and for fp32 codebooks) rq_logits is rq_build_lut + rq_lut_logits."""
    rng = np.random.default_rng(500)
    for cb in ("f32", "bf16"):
        mat = synth.gen_matrix(rng, 4000, 96, 16, 256, 2, (0.02, 0.005), cb)
        h = synth.gen_hidden(rng, 16 if cb == "f32" else 2, 96)
        W, hd = to_dev(mat), dev(h)
        assert la.logits_method(W, h.shape[0]) == la.RQ_METHOD_TABLE
        lg, am, _, _ = la.logits(W, hd, softcap=30.0)
        lg2, am2, _, _ = la.lut_logits(W, la.build_lut(W, hd), h.shape[0], softcap=30.0)
        assert torch.equal(lg, lg2) and torch.equal(am, am2)


def test_logits_packed8_uses_the_table_method():
    """8-bit codes (K <= 256) are not staged for the matrix cores: rq_logits takes the table method at any B
    and gives the two-call form's bits."""
    rng = np.random.default_rng(800)
    mat = synth.gen_matrix(rng, 3000, 96, 16, 256, 2, (0.02, 0.005), "bf16")
    h = synth.gen_hidden(rng, 16, 96)
    W, hd = to_dev(mat, "packed8"), dev(h)
    assert la.logits_method(W, 16) == la.RQ_METHOD_TABLE
    lg, am, _, _ = la.logits(W, hd, softcap=30.0)
    lg2, am2, _, _ = la.lut_logits(W, la.build_lut(W, hd), 16, softcap=30.0)
    assert torch.equal(lg, lg2) and torch.equal(am, am2)
    _, ref = oracle_head(mat, h, 30.0)
    check_logits(host(lg), ref)


def test_logits_ties_and_empty():
    """K = 1: every logit ties and the argmax is row 0 on the matrix cores too; B = 0 is a no-op."""
    rng = np.random.default_rng(600)
    mat = synth.gen_matrix(rng, 5000, 96, 16, 1, 2, (0.02, 0.005), "bf16")
    W = to_dev(mat)
    h = synth.gen_hidden(rng, 16, 96)
    lg, am, ti, _ = la.logits(W, dev(h), softcap=30.0, topk=5)
    g = host(lg)
    assert np.all(g == g[:, :1])
    assert np.all(host(am) == 0)
    assert np.array_equal(host(ti), np.tile(np.arange(5, dtype=np.int32), (16, 1)))
    lg0, _, _, _ = la.logits(W, torch.zeros((0, 96), device="cuda"), argmax=False)
    assert lg0.shape == (0, 5000)


def test_logits_one_group_epilogue_topk():
    """One code block (L*M = 8) leaves a single group, so the matrix-core kernel applies the softcap and
    emits the selection keys itself (no finish pass): logits, argmax and top-k against the oracle."""
    rng = np.random.default_rng(700)
    mat = synth.gen_matrix(rng, 4000, 48, 8, 256, 1, (0.05,), "bf16")
    h = synth.gen_hidden(rng, 24, 48)
    W = to_dev(mat)
    lg, am, ti, tv = la.logits(W, dev(h), softcap=30.0, topk=7)
    g = host(lg)
    _, ref = oracle_head(mat, h, 30.0)
    check_logits(g, ref)
    check_argmax(host(am), g, ref)
    tol = 1e-5 * np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
    check_topk(g, host(ti), host(tv), host(am), ref, tol, 7)
    _, am2, ti2, _ = la.logits(W, dev(h), softcap=30.0, logits=False, topk=7)
    assert torch.equal(am, am2) and torch.equal(ti, ti2)


@pytest.mark.parametrize("B", [3, 9])
@pytest.mark.parametrize("k", [1, 50, 1000, 1024])
def test_topk_exact_ties_ragged(B, k):
    """Top-k on exact small-integer inputs (many equal logits, so the order among ties is decided by the id)
    over 3000 rows (a last 1024-row block of 952): the ids are exactly the first k of the GPU's own logits
    sorted by (value desc, id asc), including k above a block's rows (1000, 1024) and k = 1; B=3 runs the
    table method, B=9 the matrix cores."""
    rows = 3000
    mat, h = synth.gen_exact(500 + B, rows, 96, 16, 64, 2, B, cb_dtype="bf16", cmax=2, hmax=1)
    W = to_dev(mat)
    lg, am, ti, tv = la.logits(W, dev(h), softcap=0.0, topk=k)
    g, ids, vals = host(lg), host(ti), host(tv)
    z, _ = O().logits(mat.codes, mat.codebooks, True, h, 0.0)
    assert np.array_equal(g.astype(np.float64), z)
    for b in range(B):
        order = np.lexsort((np.arange(rows), -g[b]))[:k]
        assert len(np.unique(g[b])) < rows // 4          # ties everywhere
        assert np.array_equal(ids[b], order), (b, k)
        assert np.array_equal(vals[b], g[b, order])
        assert host(am)[b] == order[0]
