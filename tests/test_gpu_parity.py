"""HIP path vs the CPU oracle, element by element, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import lut_logits_amd as la
import oracle
from lut_logits_amd import synth
from gpu_util import bf16_table_tol, check_argmax, check_logits, check_topk, dev, host, oracle_head, to_dev

pytestmark = pytest.mark.gpu

O = oracle.default


def _rand(seed, rows, D, M, K, L, cb_dtype="f32", sigmas=None):
    rng = np.random.default_rng(seed)
    sig = sigmas or tuple(0.02 * 0.25 ** l for l in range(L))
    return synth.gen_matrix(rng, rows, D, M, K, L, sig, cb_dtype), rng


# ------------------------------------------------------------------ layout

@pytest.mark.parametrize("rows,NP", [(1, 1), (63, 7), (4097, 34), (130, 768), (65, 1000)])
def test_pack_codes_bit_exact(rows, NP):
    rng = np.random.default_rng(rows + NP)
    codes = rng.integers(0, 65536, size=(rows, NP), dtype=np.uint16)
    out = host(la.pack_codes(dev(codes.view(np.int16)), rows, 1, NP)).view(np.uint16)
    NQ = (NP + 7) // 8
    padded = np.zeros((rows, 8 * NQ), np.uint16)
    padded[:, :NP] = codes
    want = padded.reshape(rows, NQ, 8).transpose(1, 0, 2).reshape(-1)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("rows,NP", [(1, 1), (63, 7), (4097, 34), (130, 768), (65, 1000)])
def test_pack_codes10_bit_exact(rows, NP):
    """The 10-bit layout against a host packing: 12 codes per 16-byte block, three per 32-bit word."""
    rng = np.random.default_rng(7 * rows + NP)
    codes = rng.integers(0, 1024, size=(rows, NP), dtype=np.uint16)
    out = host(la.pack_codes10(dev(codes.view(np.int16)), rows, 1, NP)).view(np.uint32)
    NQ = (NP + 11) // 12
    padded = np.zeros((rows, 12 * NQ), np.uint32)
    padded[:, :NP] = codes
    trip = padded.reshape(rows, NQ, 4, 3)
    words = trip[..., 0] | (trip[..., 1] << 10) | (trip[..., 2] << 20)        # [rows][NQ][4]
    assert np.array_equal(out, words.transpose(1, 0, 2).reshape(-1))


@pytest.mark.parametrize("rows,NP", [(1, 1), (63, 7), (4097, 34), (130, 768), (65, 1000)])
def test_pack_codes8_bit_exact(rows, NP):
    """The 8-bit layout against a host packing: 16 codes per 16-byte block, one byte each."""
    rng = np.random.default_rng(11 * rows + NP)
    codes = rng.integers(0, 256, size=(rows, NP), dtype=np.uint16)
    out = host(la.pack_codes8(dev(codes.view(np.int16)), rows, 1, NP)).view(np.uint8)
    NQ = (NP + 15) // 16
    padded = np.zeros((rows, 16 * NQ), np.uint8)
    padded[:, :NP] = codes
    assert np.array_equal(out, padded.reshape(rows, NQ, 16).transpose(1, 0, 2).reshape(-1))


# ------------------------------------------------------------------ row decode

@pytest.mark.parametrize("layout", ["rows", "blocked", "packed10", "packed8"])
@pytest.mark.parametrize("L,cb_dtype,out_dtype", [(2, "f32", "f32"), (2, "f32", "bf16"), (2, "bf16", "bf16"),
                                                  (3, "f32", "f32"), (4, "bf16", "f32"), (1, "f32", "f32")])
def test_decode_rows_bit_exact(layout, L, cb_dtype, out_dtype):
    mat, rng = _rand(30 + L, 4096, 96, 16, 256, L, cb_dtype)
    ids = np.concatenate([rng.integers(0, 4096, 8), [0, 4095, -1, 4096, 2 ** 31 - 1]]).astype(np.int32)
    W = to_dev(mat, layout)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = host(la.decode_rows(W, dev(ids), out_dtype, bad_ids=bad))
    want, nbad = O().decode_rows(mat.codes, mat.codebooks, mat.cb_is_bf16, ids, out_dtype == "bf16")
    if out_dtype == "bf16":
        out = out.view(np.uint16)
    assert np.array_equal(out, want)
    assert int(bad.item()) == nbad == 3


def test_decode_rows_gemma_shape():
    """64 token ids on the 256000 x 2304 head (bf16 codebooks, bf16 rows), bit-exact."""
    cfg = synth.CONFIGS["gemma_b1"]
    mat, _, ids = synth.make_head(cfg)
    W = to_dev(mat)
    out = host(la.decode_rows(W, dev(ids), "bf16")).view(np.uint16)
    want, nbad = O().decode_rows(mat.codes, mat.codebooks, True, ids, True)
    assert nbad == 0 and np.array_equal(out, want)


@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_decode_rows_code_out_of_range(layout):
    """A code equal to K (a broken precondition) decodes as codeword K-1 instead of reading past the
    codebook: placed only at pair (0, 0) of one row, so even an unclamped read would stay inside the
    codebook array. Every other element and row is the oracle's."""
    mat, rng = _rand(41, 256, 96, 16, 64, 2, "f32")
    bad_codes = mat.codes.copy()
    bad_codes[5, 0, 0] = mat.K
    bad = synth.RQMatrix(mat.rows, mat.D, mat.M, mat.d, mat.K, mat.L, mat.cb_dtype, mat.codebooks, bad_codes)
    W = to_dev(bad, layout)
    ids = np.array([5, 6], np.int32)
    out = host(la.decode_rows(W, dev(ids)))
    fixed = bad_codes.copy()
    fixed[5, 0, 0] = mat.K - 1
    want, _ = O().decode_rows(fixed, mat.codebooks, False, ids, False)
    assert np.array_equal(out, want)


# ------------------------------------------------------------------ table build

@pytest.mark.parametrize("cb_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B", [1, 3, 16])
def test_build_lut(cb_dtype, B):
    mat, rng = _rand(40 + B, 8, 96, 16, 256, 2, cb_dtype)
    h = synth.gen_hidden(rng, B, 96)
    W = to_dev(mat)
    lut = host(la.build_lut(W, dev(h))).reshape(2, 16, 256, B)
    ref = O().build_lut(mat.codebooks, mat.cb_is_bf16, h).transpose(1, 2, 3, 0)   # [L][M][K][B]
    # d=6 fp32 FMAs: error <= 6 * 2^-24 * sum_j |a_j c_j|
    cbf = mat.codebooks_f32().astype(np.float64)
    bound = np.einsum("bmj,lmkj->lmkb", np.abs(h.astype(np.float64)).reshape(B, 16, 6), np.abs(cbf)) * 6 * 2.0 ** -24
    assert np.all(np.abs(lut - ref) <= bound + 1e-30)


def test_build_lut_exact_and_bf16_table():
    mat, h = synth.gen_exact(7, rows=4, D=96, M=16, K=256, L=2, B=2)
    W = to_dev(mat)
    lut = host(la.build_lut(W, dev(h))).reshape(2, 16, 256, 2)
    ref = O().build_lut(mat.codebooks, False, h).transpose(1, 2, 3, 0)
    assert np.array_equal(lut, ref)
    lutb = host(la.build_lut(W, dev(h), lut_dtype="bf16")).view(np.uint16).reshape(2, 16, 256, 2)
    # exact fp32 values, then one rounding to bf16 (nearest even)
    assert np.array_equal(lutb, synth.f32_to_bf16_bits(ref.astype(np.float32)))


@pytest.mark.parametrize("cb_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lut_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,d,K", [(8, 6, 300), (24, 3, 300), (64, 6, 300), (12, 8, 300), (16, 3, 301)])
def test_build_lut_batched_exact(cb_dtype, lut_dtype, B, d, K):
    """Batched tables on exact inputs, with a partial last tile of codewords (K=300, 301 over tiles of 256): the
    fp32 table equals the oracle's and the bf16 one is its single rounding (nearest even). B=8, 64 and 16 fill whole
    16-byte units of entries per lane of a codeword (both table types); B=24 and B=12 do not divide the workgroup
    that way and take the per-codeword loop, as do bf16 codebooks at d=3, K=301, whose tiles are not whole 4-byte
    words."""
    M = 96 // d
    mat, h = synth.gen_exact(60 + B + d + K, rows=4, D=96, M=M, K=K, L=2, B=B, cb_dtype=cb_dtype)
    W = to_dev(mat)
    lut = host(la.build_lut(W, dev(h), lut_dtype=lut_dtype))
    ref = O().build_lut(mat.codebooks, mat.cb_is_bf16, h).transpose(1, 2, 3, 0)   # [L][M][K][B]
    if lut_dtype == "f32":
        assert np.array_equal(lut.reshape(2, M, K, B), ref)
    else:
        assert np.array_equal(lut.view(np.uint16).reshape(2, M, K, B), synth.f32_to_bf16_bits(ref.astype(np.float32)))


def test_build_lut_gelu_prologue():
    mat, rng = _rand(50, 8, 96, 48, 64, 2)
    g = synth.gen_hidden(rng, 2, 96) * np.float32(2.0)
    u = synth.gen_hidden(rng, 2, 96)
    W = to_dev(mat)
    lut = host(la.build_lut(W, dev(g), x2=dev(u), prologue=la.RQ_PRO_GELU_TANH_MUL)).reshape(2, 48, 64, 2)
    a = O().gelu_mul(g.astype(np.float64), u.astype(np.float64))
    ref = O().build_lut(mat.codebooks, False, a).transpose(1, 2, 3, 0)
    scale = np.abs(ref).max()
    assert np.abs(lut - ref).max() <= 1e-5 * scale


# ------------------------------------------------------------------ logits: exact arithmetic

EXACT_SHAPES = [
    # rows, D, M, K, L, B
    (4097, 96, 16, 256, 2, 1),
    (4097, 102, 17, 1000, 2, 1),    # odd M, K not a power of two, ragged rows
    (1, 6, 1, 1, 1, 1),             # one row, one codeword, one pair
    (300, 34, 17, 5, 1, 2),         # L*M not a multiple of 8 (blocked layout only), ragged batch tile
    (2049, 96, 16, 256, 2, 16),
    (1500, 96, 16, 128, 3, 17),     # batch 16 + ragged 1
    (700, 96, 96, 64, 2, 5),        # d = 1
    (333, 64, 1, 512, 2, 3),        # M = 1, d = D
    (4500, 2304, 384, 1000, 2, 1),  # the Gemma head's pairs: the pipelined kernel (16- and 10-bit codes)
    (5000, 1536, 256, 64, 2, 1),    # 512 pairs, K = 64: the pipelined kernel on 16-bit codes
    (4500, 2304, 384, 1001, 2, 1),  # K % 4 != 0: a pair's table is no whole number of 16-byte words
]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["rows", "blocked", "packed10", "packed8"])
def test_lut_logits_exact(shape, layout):
    """Small-integer inputs: every fp32 step is exact, so logits (softcap off) equal the oracle bit for bit."""
    rows, D, M, K, L, B = shape
    if layout == "rows" and (L * M) % 8:
        pytest.skip("row-major codes need L*M % 8 == 0")
    if (layout == "packed10" and K > 1024) or (layout == "packed8" and K > 256):
        pytest.skip("K too large for the packed layout")
    mat, h = synth.gen_exact(rows + K, rows, D, M, K, L, B)
    W = to_dev(mat, layout)
    lut = la.build_lut(W, dev(h))
    lg, am, _, _ = la.lut_logits(W, lut, B, softcap=0.0)
    z, _ = O().logits(mat.codes, mat.codebooks, False, h, 0.0)
    got = host(lg)
    assert np.array_equal(got.astype(np.float64), z)
    assert np.array_equal(host(am), np.argmax(got, axis=1).astype(np.int32))


def test_lut_logits_bf16_codebooks_exact():
    mat, h = synth.gen_exact(3, 2500, 96, 16, 300, 2, 4, cb_dtype="bf16")
    W = to_dev(mat)
    lg, _, _, _ = la.lut_logits(W, la.build_lut(W, dev(h)), 4, softcap=0.0)
    z, _ = O().logits(mat.codes, mat.codebooks, True, h, 0.0)
    assert np.array_equal(host(lg).astype(np.float64), z)


@pytest.mark.parametrize("lut_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B", [20, 24, 40])
def test_lut_logits_batch_tiled_exact(B, lut_dtype):
    """Batches the lookup+sum splits into batch tiles (fp32 tables: 16 + the rest; bf16 tables: tiles of 4), so
    the call first copies the table into the batch-tiled layout: 16-byte units where a table row is whole 16-byte
    units (all but B=20 with a bf16 table, which takes the 4-byte copy), a last block of 32 of 64 table rows
    (K=501), and zero columns past B. Exact inputs: every table entry is exact in bf16 too, so the logits equal the
    oracle's bit for bit."""
    mat, h = synth.gen_exact(900 + B, 1500, 96, 16, 501, 2, B)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h), lut_dtype=lut_dtype)
    lg, am, _, _ = la.lut_logits(W, lut, B, softcap=0.0, lut_dtype=lut_dtype)
    z, _ = O().logits(mat.codes, mat.codebooks, False, h, 0.0)
    got = host(lg)
    assert np.array_equal(got.astype(np.float64), z)
    assert np.array_equal(host(am), np.argmax(got, axis=1).astype(np.int32))


@pytest.mark.parametrize("B,rows", [(24, 20000), (40, 9000), (4, 12000)])
def test_lut_logits_row_sets_exact(B, rows):
    """bf16 tables in several batch tiles of 4 over more than two slabs of 4,096 rows: each workgroup runs two row
    sets per staged chunk (slabs of 8,192 rows, the last one ragged), and B=4 (a single tile) keeps one. Exact
    inputs: the logits equal the oracle's bit for bit."""
    mat, h = synth.gen_exact(700 + B, rows, 96, 16, 301, 2, B)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h), lut_dtype="bf16")
    lg, am, _, _ = la.lut_logits(W, lut, B, softcap=0.0, lut_dtype="bf16")
    z, _ = O().logits(mat.codes, mat.codebooks, False, h, 0.0)
    got = host(lg)
    assert np.array_equal(got.astype(np.float64), z)
    assert np.array_equal(host(am), np.argmax(got, axis=1).astype(np.int32))


@pytest.mark.parametrize("B", [16, 17])
def test_lut_logits_fp32_row_sets_exact(B):
    """fp32 tables of 16 vectors: two row sets per workgroup (slabs of 2 x 4 x 256 rows) with groups of pairs
    added to keep a workgroup per CU. 5000 rows span three slabs, the last one ragged; B=17 adds a second,
    one-vector batch tile. The plan query confirms the route; exact inputs make the logits the oracle's bit
    for bit."""
    mat, h = synth.gen_exact(750 + B, 5000, 96, 16, 301, 2, B)
    W = to_dev(mat)
    plan = la.lut_logits_plan(W, B, "f32")
    assert plan["BT"] == 16 and plan["rset"] == 2 and plan["G"] > 1 and plan["S"] == 3, plan
    assert plan["NBT"] == (B + 15) // 16
    lut = la.build_lut(W, dev(h))
    lg, am, _, _ = la.lut_logits(W, lut, B, softcap=0.0)
    z, _ = O().logits(mat.codes, mat.codebooks, False, h, 0.0)
    got = host(lg)
    assert np.array_equal(got.astype(np.float64), z)
    assert np.array_equal(host(am), np.argmax(got, axis=1).astype(np.int32))


# ------------------------------------------------------------------ logits: float parity

def test_tiny_config():
    """The tiny RQ head: V=4096, D=96, M=16, K=256, L=2, fp32 codebooks, softcap 30, argmax, 8 decoded rows."""
    cfg = synth.CONFIGS["tiny"]
    mat, h, ids = synth.make_head(cfg)
    for layout in ("rows", "blocked", "packed10", "packed8"):
        W = to_dev(mat, layout)
        lg, am, _, _ = la.lut_logits(W, la.build_lut(W, dev(h)), 1, softcap=cfg.softcap)
        _, ref = oracle_head(mat, h, cfg.softcap)
        check_logits(host(lg), ref)
        check_argmax(host(am), host(lg), ref)
        rows = host(la.decode_rows(W, dev(ids)))
        want, _ = O().decode_rows(mat.codes, mat.codebooks, False, ids, False)
        assert np.array_equal(rows, want)


@pytest.mark.parametrize("B", [1, 2, 16, 20])
def test_float_parity_batched(B):
    mat, rng = _rand(60 + B, 3000, 96, 16, 512, 2, "bf16")
    h = synth.gen_hidden(rng, B, 96)
    W = to_dev(mat)
    lg, am, _, _ = la.lut_logits(W, la.build_lut(W, dev(h)), B, softcap=30.0)
    _, ref = oracle_head(mat, h, 30.0)
    check_logits(host(lg), ref)
    check_argmax(host(am), host(lg), ref)


def test_argmax_ties_lowest_index():
    """K = 1: every row decodes to the same vector, every logit ties, the argmax is row 0."""
    mat, rng = _rand(70, 5000, 96, 16, 1, 2)
    h = synth.gen_hidden(rng, 3, 96)
    W = to_dev(mat)
    lg, am, ti, _ = la.lut_logits(W, la.build_lut(W, dev(h)), 3, softcap=30.0, topk=5)
    g = host(lg)
    assert np.all(g == g[:, :1])
    assert list(host(am)) == [0, 0, 0]
    assert np.array_equal(host(ti), np.tile(np.arange(5, dtype=np.int32), (3, 1)))


def test_no_logits_output_and_determinism():
    mat, rng = _rand(80, 9000, 96, 16, 256, 2)
    h = synth.gen_hidden(rng, 1, 96)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h))
    lg1, am1, _, _ = la.lut_logits(W, lut, 1)
    lg2, am2, _, _ = la.lut_logits(W, lut, 1)
    _, am3, _, _ = la.lut_logits(W, lut, 1, logits=False)
    assert torch.equal(lg1, lg2) and torch.equal(am1, am2) and torch.equal(am1, am3)


def test_output_canaries():
    """Nothing outside [B][rows] of the logits buffer is written."""
    mat, rng = _rand(81, 1000, 96, 16, 256, 2)
    h = synth.gen_hidden(rng, 2, 96)
    W = to_dev(mat)
    buf = torch.full((2 * 1000 + 64,), float("nan"), device="cuda")
    la.lut_logits(W, la.build_lut(W, dev(h)), 2, out=buf[:2000].view(2, 1000))
    tail = host(buf[2000:])
    assert np.all(np.isnan(tail))
    assert not np.any(np.isnan(host(buf[:2000])))


def test_empty_work_is_noop():
    mat, rng = _rand(82, 10, 96, 16, 16, 2)
    W = to_dev(mat)
    h = torch.zeros((0, 96), device="cuda")
    lut = la.build_lut(W, h)
    assert lut.numel() == 0
    out = la.decode_rows(W, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 96)


# ------------------------------------------------------------------ top-k with bf16 tables

@pytest.mark.parametrize("lut_dtype", ["f32", "bf16"])
def test_topk(lut_dtype):
    K, L, B, k = 4096, 4, 5, 50
    mat, rng = _rand(90, 6000, 96, 16, K, L, "bf16", sigmas=(0.02, 0.008, 0.003, 0.001))
    h = synth.gen_hidden(rng, B, 96)
    W = to_dev(mat)
    lut = la.build_lut(W, dev(h), lut_dtype=lut_dtype)
    lg, am, ti, tv = la.lut_logits(W, lut, B, softcap=30.0, lut_dtype=lut_dtype, topk=k)
    g = host(lg)
    _, ref = oracle_head(mat, h, 30.0)
    if lut_dtype == "bf16":
        tolv = bf16_table_tol(mat, h, ref)
        check_logits(g, ref, tol=tolv.max(axis=1))
    else:
        tolv = 1e-5 * np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
        check_logits(g, ref)
    check_topk(g, host(ti), host(tv), host(am), ref, tolv, k)


# ------------------------------------------------------------------ MLP LUT-matvec

def test_lut_matvec_small_chain():
    rng = np.random.default_rng(100)
    hid, inter = 96, 160
    gate = synth.gen_matrix(rng, inter, hid, 48, 64, 2, (0.02, 0.005), "f32")
    up = synth.gen_matrix(rng, inter, hid, 48, 64, 2, (0.02, 0.005), "f32")
    down = synth.gen_matrix(rng, hid, inter, 80, 64, 2, (0.02, 0.005), "f32")
    x = synth.gen_hidden(rng, 2, hid)
    Wg, Wu, Wd = to_dev(gate), to_dev(up), to_dev(down)
    g = la.lut_matvec(Wg, dev(x))
    u = la.lut_matvec(Wu, dev(x))
    y = la.lut_matvec(Wd, g, x2=u, prologue=la.RQ_PRO_GELU_TANH_MUL)
    og, ou, oa, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                             (down.codes, down.codebooks, False), x)
    check_logits(host(g), og)
    check_logits(host(u), ou)
    check_logits(host(y), oy)


@pytest.mark.parametrize("d", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", ["rows", "blocked", "packed10", "packed8"])
def test_lut_matvec_fused_build_exact(d, layout):
    """One activation vector with fp32 codebooks: the table is built while staging. Exact inputs, ragged rows
    and (blocked layout) a partly empty last code block: bit-exact against the oracle."""
    D = 120
    M = D // d
    if layout == "rows" and (2 * M) % 8:
        pytest.skip("row-major codes need L*M % 8 == 0")
    mat, x = synth.gen_exact(40 + d, 3001, D, M, 256, 2, 1)
    W = to_dev(mat, layout)
    y = la.lut_matvec(W, dev(x))
    assert np.array_equal(host(y).astype(np.float64), O().matvec(mat.codes, mat.codebooks, False, x))


@pytest.mark.parametrize("rows,D,K,layout", [
    (5000, 1004, 256, "blocked"),   # 1004 pairs: a partly empty last code block of 8
    (5000, 1004, 256, "packed10"),  # ... and of 12
    (4097, 2304, 1024, "packed10"), # one row past four slabs of 1024
    (9216, 2304, 1024, "blocked"),  # the MLP gate's shape
    (6000, 520, 64, "blocked"),     # 520 pairs (65 blocks), K = 64
    (6000, 100, 256, "blocked"),    # 13 blocks of pairs: the one-buffer kernel
    (3001, 100, 256, "blocked"),    # one slab: the one-buffer kernel
    (1, 2304, 1024, "blocked"),     # one row
    (37, 4608, 1024, "packed10"),   # the MLP down's width, few rows
    (700, 600, 2048, "blocked"),    # K > 1024
])
def test_lut_matvec_fused_d2_exact(rows, D, K, layout):
    """The fused build at d = 2. Matrices taller than one slab (4096 rows) with 16- or 10-bit codes, K <= 1024
    and at least 64 blocks of pairs take the pipelined kernel (one code block per chunk, two chunks in flight,
    chunks split evenly over the groups); the others the one-buffer kernel. Exact inputs, bit-exact against
    the oracle."""
    mat, x = synth.gen_exact(rows + D + K, rows, D, D // 2, K, 2, 1)
    W = to_dev(mat, layout)
    y = la.lut_matvec(W, dev(x))
    assert np.array_equal(host(y).astype(np.float64), O().matvec(mat.codes, mat.codebooks, False, x))


def test_lut_matvec_fused_build_gelu_and_fallback():
    """The GELU*up prologue feeding the fused build, and a row width whose activation vector does not fit
    beside a table chunk in LDS (the separate table build is used instead)."""
    rng = np.random.default_rng(120)
    for rows, D, M, K in ((2500, 128, 64, 256), (300, 40000, 20000, 16)):
        mat = synth.gen_matrix(rng, rows, D, M, K, 2, (0.02, 0.005), "f32")
        g = synth.gen_hidden(rng, 1, D)
        u = synth.gen_hidden(rng, 1, D)
        W = to_dev(mat)
        y = la.lut_matvec(W, dev(g), x2=dev(u), prologue=la.RQ_PRO_GELU_TANH_MUL)
        a = O().gelu_mul(g.astype(np.float64), u.astype(np.float64))
        check_logits(host(y), O().matvec(mat.codes, mat.codebooks, False, a))


def test_mlp_layer_gemma_shapes():
    """One Gemma-2-2B MLP layer: gate/up 9216x2304 (d=2), down 2304x9216 (d=2), K=1024, L=2, fp32 codebooks."""
    gate, up, down = synth.make_mlp_layer(0)
    x = synth.make_mlp_x()
    Wg, Wu, Wd = to_dev(gate), to_dev(up), to_dev(down)
    g = la.lut_matvec(Wg, dev(x))
    u = la.lut_matvec(Wu, dev(x))
    y = la.lut_matvec(Wd, g, x2=u, prologue=la.RQ_PRO_GELU_TANH_MUL)
    og, ou, oa, oy = O().mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                             (down.codes, down.codebooks, False), x)
    check_logits(host(g), og)
    check_logits(host(u), ou)
    check_logits(host(y), oy)
    # down alone, fed the oracle's gate/up outputs rounded to fp32
    g32, u32 = og.astype(np.float32), ou.astype(np.float32)
    y1 = la.lut_matvec(Wd, dev(g32), x2=dev(u32), prologue=la.RQ_PRO_GELU_TANH_MUL)
    a = O().gelu_mul(g32.astype(np.float64), u32.astype(np.float64))
    check_logits(host(y1), O().matvec(down.codes, down.codebooks, False, a))


# ------------------------------------------------------------------ dense comparison head

@pytest.mark.parametrize("rows,D", [(1, 8), (16, 32), (33, 40), (300, 2304), (1001, 104)])
def test_pack_dense_layout(rows, D):
    """rq_pack_dense: Et[tile][kstep][i][j] = E[16 tile + i][32 kstep + j], zero past rows and D, byte-exact
    against the layout written out in numpy (row and column counts that are and are not whole tiles)."""
    rng = np.random.default_rng(rows * 7 + D)
    E = rng.integers(-32768, 32768, size=(rows, D), dtype=np.int64).astype(np.int16)
    head = la.pack_dense(dev(E))
    nt, ks = (rows + 15) // 16, (D + 31) // 32
    P = np.zeros((nt * 16, ks * 32), np.int16)
    P[:rows, :D] = E
    want = P.reshape(nt, 16, ks, 32).transpose(0, 2, 1, 3).reshape(-1)
    assert head.nbytes == la.dense_tiled_bytes(rows, D) == want.size * 2
    assert np.array_equal(host(head.tiles), want)


@pytest.mark.parametrize("B,D,rows", [(1, 96, 5000), (3, 96, 5000), (16, 96, 5000), (17, 96, 5000), (40, 200, 5000),
                                      (128, 96, 5000), (128, 600, 5000), (5, 200, 4993), (70, 104, 1001),
                                      (2, 2304, 300)])
def test_dense_comparator(B, D, rows):
    """The dense bf16 head (GEMV at B=1, matrix-core GEMM up to B=128, with h staged in chunks of columns for
    B > 16) against an fp64 numpy product of the same bf16 values: every logit, the softcap, and the argmax as
    the first maximum of the GPU's own logits. Ragged cases: a last block of 256 rows cut short (5000), a last
    tile of 16 rows cut short (4993, 1001), D not a multiple of 32 (200, 104: zero-padded k-steps)."""
    M = D // 6 if D % 6 == 0 else D // 8
    mat, rng = _rand(110 + B + rows, rows, D, M, 256, 2, "bf16")
    h = synth.gen_hidden(rng, B, D)
    W = to_dev(mat)
    E = la.decode_rows(W, torch.arange(rows, dtype=torch.int32, device="cuda"), "bf16")
    lg, am = la.dense_logits(la.pack_dense(E), dev(h), softcap=30.0)
    Ef = synth.bf16_bits_to_f32(host(E).view(np.uint16)).astype(np.float64)
    hb = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(h)).astype(np.float64)
    ref = 30.0 * np.tanh((hb @ Ef.T) / 30.0)
    check_logits(host(lg), ref)
    assert np.array_equal(host(am), np.argmax(host(lg), axis=1).astype(np.int32))
