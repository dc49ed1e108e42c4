"""Pins that tie the CPU oracle to facts outside itself.

Every function takes an oracle instance and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix. The same battery
runs against the real oracle (every pin must hold) and against deliberately
broken copies of it (at least one pin must fail), see test_oracle_mutants.py.

Sources of truth used here, none of which is the oracle's own code:
  - exact rational arithmetic on inputs where fp64 makes no rounding;
  - identities of the method: the lookup+sum form equals decode+matmul
    (runtime-compression page, correctness-check table), residual levels add,
    relabelling codewords or permuting subspaces changes nothing, linearity;
  - special cases that reduce to numpy / torch library routines (gather,
    matmul, sort, argmax, bf16 conversion, GELU with the tanh approximation);
  - closed values of tanh and GELU.
"""
import math
from fractions import Fraction

import numpy as np
import torch

from lut_logits_amd import synth


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / scale


def _random_matrix(seed, rows, D, M, K, L, cb_dtype="f32", sigmas=None):
    rng = np.random.default_rng(seed)
    sig = sigmas or tuple(0.02 / (2 ** l) for l in range(L))
    return synth.gen_matrix(rng, rows, D, M, K, L, sig, cb_dtype), rng


# --------------------------------------------------------------------------- logits

def pin_exact_rational_logits(o):
    """Small-integer inputs: fp64 makes no rounding, so the oracle must equal the
    exact rational value of sum_{l,m} <h_m, C[l][m][code]> (the lookup+sum form,
    evaluated with Python Fractions)."""
    for (rows, D, M, K, L) in [(37, 12, 4, 5, 2), (19, 9, 9, 3, 3), (11, 8, 1, 7, 1)]:
        mat, h = synth.gen_exact(seed=rows, rows=rows, D=D, M=M, K=K, L=L, B=2)
        z, _ = o.logits(mat.codes, mat.codebooks, False, h, 0.0)
        d = D // M
        cbq = [[[[Fraction(float(mat.codebooks[l, m, k, j])) for j in range(d)] for k in range(K)]
                 for m in range(M)] for l in range(L)]
        for b in range(h.shape[0]):
            hq = [Fraction(float(v)) for v in h[b]]
            for r in range(rows):
                total = Fraction(0)
                for m in range(M):
                    for l in range(L):
                        cw = cbq[l][m][int(mat.codes[r, l, m])]
                        total += sum(hq[m * d + j] * cw[j] for j in range(d))
                assert Fraction(float(z[b, r])) == total, (rows, b, r)


def pin_lut_equals_decode(o):
    """The page's correctness gate (lookup+sum vs direct decode+matmul), in fp64."""
    for (rows, D, M, K, L, cbd) in [(300, 24, 4, 16, 2, "f32"), (257, 18, 6, 33, 3, "bf16"), (64, 5, 5, 2, 1, "f32")]:
        mat, rng = _random_matrix(rows + K, rows, D, M, K, L, cbd)
        h = synth.gen_hidden(rng, 3, D)
        z, _ = o.logits(mat.codes, mat.codebooks, mat.cb_is_bf16, h, 0.0)
        lut = o.build_lut(mat.codebooks, mat.cb_is_bf16, h)
        assert lut.shape == (3, L, M, K)
        z2 = o.lut_sum(mat.codes, lut)
        assert _rel(z2, z) <= 1e-12


def pin_single_subspace_is_matmul(o):
    """M=1, L=1 (d = D): the decoded matrix is the codebook gathered by code; logits = numpy matmul."""
    mat, rng = _random_matrix(5, 200, 16, 1, 50, 1)
    h = synth.gen_hidden(rng, 2, 16)
    z, _ = o.logits(mat.codes, mat.codebooks, False, h, 0.0)
    E = mat.codebooks[0, 0][mat.codes[:, 0, 0].astype(np.int64)].astype(np.float64)
    assert _rel(z, h.astype(np.float64) @ E.T) <= 1e-13


def pin_scalar_subspaces_gather(o):
    """d=1 (M = D): W[r][m] = sum_l C[l][m][code[r][l][m]][0], built with numpy fancy indexing."""
    rows, D, K, L = 150, 10, 9, 2
    mat, rng = _random_matrix(6, rows, D, D, K, L)
    h = synth.gen_hidden(rng, 2, D)
    z, _ = o.logits(mat.codes, mat.codebooks, False, h, 0.0)
    W = np.zeros((rows, D))
    for l in range(L):
        W += mat.codebooks[l, np.arange(D)[None, :], mat.codes[:, l, :].astype(np.int64), 0]
    assert _rel(z, h.astype(np.float64) @ W.T) <= 1e-13


def pin_levels_add(o):
    """Residual levels add: logits of an L-level matrix = sum of the logits of each level alone."""
    mat, rng = _random_matrix(7, 120, 12, 3, 11, 3)
    h = synth.gen_hidden(rng, 2, 12)
    z, _ = o.logits(mat.codes, mat.codebooks, False, h, 0.0)
    parts = sum(o.logits(mat.codes[:, l:l + 1, :], mat.codebooks[l:l + 1], False, h, 0.0)[0] for l in range(3))
    assert _rel(parts, z) <= 1e-13


def pin_codeword_relabelling(o):
    """Permuting the codewords of each (l,m) and remapping the codes leaves logits bit-identical."""
    rows, D, M, K, L = 90, 12, 4, 13, 2
    mat, rng = _random_matrix(8, rows, D, M, K, L)
    h = synth.gen_hidden(rng, 2, D)
    z, _ = o.logits(mat.codes, mat.codebooks, False, h, 0.0)
    cb2 = np.empty_like(mat.codebooks)
    codes2 = np.empty_like(mat.codes)
    for l in range(L):
        for m in range(M):
            perm = rng.permutation(K)            # new slot s holds old codeword perm[s]
            cb2[l, m] = mat.codebooks[l, m, perm]
            inv = np.argsort(perm)               # old code c lives at new slot inv[c]
            codes2[:, l, m] = inv[mat.codes[:, l, m]]
    z2, _ = o.logits(codes2, cb2, False, h, 0.0)
    assert np.array_equal(z, z2)


def pin_subspace_permutation(o):
    """Reordering the subspaces consistently in h, codebooks and codes leaves logits unchanged."""
    rows, D, M, K, L = 80, 15, 5, 7, 2
    mat, rng = _random_matrix(9, rows, D, M, K, L)
    d = D // M
    h = synth.gen_hidden(rng, 2, D)
    z, _ = o.logits(mat.codes, mat.codebooks, False, h, 0.0)
    sigma = rng.permutation(M)
    h2 = h.reshape(2, M, d)[:, sigma, :].reshape(2, D)
    z2, _ = o.logits(mat.codes[:, :, sigma], mat.codebooks[:, sigma], False, h2, 0.0)
    assert _rel(z2, z) <= 1e-13


def pin_linear_in_h(o):
    """Logits are linear in h (h1 and h2 on disjoint coordinates, so 0.5*h1 + 0.25*h2 is exact in fp32)."""
    mat, rng = _random_matrix(10, 70, 8, 4, 6, 2)
    mask = (np.arange(8) % 3 == 0).astype(np.float32)
    h1 = synth.gen_hidden(rng, 1, 8) * mask
    h2 = synth.gen_hidden(rng, 1, 8) * (1 - mask)
    z1, _ = o.logits(mat.codes, mat.codebooks, False, h1, 0.0)
    z2, _ = o.logits(mat.codes, mat.codebooks, False, h2, 0.0)
    z12, _ = o.logits(mat.codes, mat.codebooks, False, (h1.astype(np.float64) * 0.5 + h2 * 0.25).astype(np.float32), 0.0)
    assert _rel(z12, 0.5 * z1 + 0.25 * z2) <= 1e-12


def pin_unit_vector_reads_decode(o):
    """h = e_i makes z[r] = W[r][i]: logits and row decode agree on every element."""
    mat, _ = _random_matrix(11, 40, 6, 3, 5, 2)
    rows_dec, _ = o.decode_rows(mat.codes, mat.codebooks, False, np.arange(40), False)
    H = np.eye(6, dtype=np.float32)
    z, _ = o.logits(mat.codes, mat.codebooks, False, H, 0.0)
    assert np.array_equal(z.T.astype(np.float32), rows_dec)


# --------------------------------------------------------------------------- softcap

def pin_softcap(o):
    """Gemma-2 final-logit softcap c*tanh(z/c) (runtime-compression page, LUT-serving paragraph):
    closed values, oddness, bound, and math.tanh; c <= 0 switches it off."""
    c = 30.0
    assert o.softcap(0.0, c) == 0.0
    assert abs(o.softcap(c * math.atanh(0.5), c) - 15.0) < 1e-12
    zs = np.array([-500.0, -31.0, -1.0, -1e-3, 2e-3, 0.7, 29.0, 77.0])
    got = o.softcap(zs, c)
    assert np.allclose(got, [c * math.tanh(z / c) for z in zs], rtol=0, atol=1e-13)
    assert np.allclose(o.softcap(-zs, c), -got, rtol=0, atol=0)
    assert np.all(np.abs(got) < c)
    assert abs(o.softcap(1e-6, c) - 1e-6) < 1e-20
    assert np.array_equal(o.softcap(zs, 0.0), zs)
    assert np.array_equal(o.softcap(zs, -1.0), zs)
    # the head applies it: logits = softcap(z)
    mat, rng = _random_matrix(12, 50, 6, 2, 4, 2)
    h = synth.gen_hidden(rng, 1, 6) * np.float32(400.0)
    z, lg = o.logits(mat.codes, mat.codebooks, False, h, c)
    assert np.allclose(lg, c * np.tanh(z / c), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- selection

def pin_argmax(o):
    """Lowest index among equal maxima, as numpy.argmax returns it."""
    rng = np.random.default_rng(13)
    x = rng.integers(0, 5, size=(6, 200)).astype(np.float64)
    assert np.array_equal(o.argmax(x), np.argmax(x, axis=1).astype(np.int32))
    y = np.full((2, 9), -3.0)
    y[0, [2, 7]] = 4.0
    y[1, 8] = 1.0
    assert list(o.argmax(y)) == [2, 8]
    # K = 1: every row decodes to the same vector, every logit ties, the answer is id 0
    mat, rng = _random_matrix(14, 33, 6, 3, 1, 2)
    h = synth.gen_hidden(rng, 2, 6)
    _, lg = o.logits(mat.codes, mat.codebooks, False, h, 30.0)
    assert np.all(lg == lg[:, :1])
    assert list(o.argmax(lg)) == [0, 0]


def pin_topk(o):
    """Order by value descending then id ascending, as a numpy lexsort gives it."""
    rng = np.random.default_rng(15)
    x = rng.integers(0, 30, size=(4, 500)).astype(np.float64)
    ids, vals = o.topk(x, 50)
    for b in range(4):
        order = np.lexsort((np.arange(500), -x[b]))[:50]
        assert np.array_equal(ids[b], order)
        assert np.array_equal(vals[b], x[b, order])
    ids1, _ = o.topk(x, 1)
    assert np.array_equal(ids1[:, 0], o.argmax(x))


# --------------------------------------------------------------------------- row decode

def pin_decode_rows(o):
    """On-demand row decode (LUT-serving paragraph): L=1 is a plain codebook gather; L=2 in fp32 is
    the correctly rounded sum of two gathered codewords (numpy float32 add); bf16 output is
    torch's round-to-nearest-even of that fp32 row; bad ids give zero rows and are counted."""
    rows, D, M, K = 64, 12, 4, 9
    mat, rng = _random_matrix(16, rows, D, M, K, 2)
    ids = np.array([0, 63, 5, 5, 17], np.int32)
    d = D // M
    g0 = mat.codebooks[0, np.arange(M)[None, :], mat.codes[ids, 0, :].astype(np.int64)].reshape(len(ids), D)
    g1 = mat.codebooks[1, np.arange(M)[None, :], mat.codes[ids, 1, :].astype(np.int64)].reshape(len(ids), D)
    out, bad = o.decode_rows(mat.codes[:, :1], mat.codebooks[:1], False, ids, False)
    assert bad == 0 and np.array_equal(out, g0)
    out, bad = o.decode_rows(mat.codes, mat.codebooks, False, ids, False)
    assert np.array_equal(out, (g0 + g1).astype(np.float32))
    outb, _ = o.decode_rows(mat.codes, mat.codebooks, False, ids, True)
    ref = torch.from_numpy(g0 + g1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(outb, ref)
    out3, _ = o.decode_rows(mat.codes, mat.codebooks, False, np.array([3], np.int32), False)
    out, bad = o.decode_rows(mat.codes, mat.codebooks, False, np.array([-1, 64, 3], np.int32), False)
    assert bad == 2 and not out[:2].any() and np.array_equal(out[2], out3[0])
    assert out.shape == (3, M * d)


def _round_to_f32(q):
    """Correct rounding (to nearest, ties to even) of an exact rational to fp32, in integer
    arithmetic: no intermediate float, so no double rounding."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** max(e - 23, -149)
    n, rem = divmod(a, ulp)
    n = int(n)
    if rem * 2 > ulp or (rem * 2 == ulp and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n * ulp))   # n * ulp is an fp32 value: float() is exact


def pin_decode_rows_many_levels(o):
    """Decoded rows for L >= 3 are the correctly rounded fp32 value of the exact level sum (one
    rounding; Python Fractions), not a level-by-level fp32 sum: a hand case where the two differ
    (1 + 2^-24 + 2^-24: fp32 sum 1, exact 1 + 2^-23), then random codebooks at L=3 and L=4 with
    codewords of very different scales, where at least one element tells the two readings apart.
    bf16 output is the nearest-even bf16 of that fp32 value."""
    cb = np.zeros((3, 1, 2, 1), np.float32)
    cb[:, 0, 0, 0] = [1.0, 2.0 ** -24, 2.0 ** -24]
    cb[:, 0, 1, 0] = [2.0 ** -24, 2.0 ** -24, 1.0]
    codes = np.zeros((2, 3, 1), np.uint16)
    codes[1] = 1
    out, _ = o.decode_rows(codes, cb, False, np.array([0, 1], np.int32), False)
    assert out[0, 0] == np.float32(1.0 + 2.0 ** -23) and out[1, 0] == np.float32(1.0 + 2.0 ** -23)
    differ = 0
    for L, seed in ((3, 31), (4, 32)):
        sig = (0.5, 3e-5, 2e-9, 1e-6)[:L]
        mat, _ = _random_matrix(seed, 40, 12, 4, 6, L, sigmas=sig)
        ids = np.arange(40, dtype=np.int32)
        got, _ = o.decode_rows(mat.codes, mat.codebooks, False, ids, False)
        gotb, _ = o.decode_rows(mat.codes, mat.codebooks, False, ids, True)
        d = mat.d
        for i in ids:
            for m in range(mat.M):
                for j in range(d):
                    vals = [mat.codebooks[l, m, mat.codes[i, l, m], j] for l in range(L)]
                    want = _round_to_f32(sum(Fraction(float(v)) for v in vals))
                    assert got[i, m * d + j] == want, (L, i, m, j)
                    seq = np.float32(0.0)
                    for v in vals:
                        seq = np.float32(seq + v)
                    differ += int(seq != want)
        wantb = torch.from_numpy(got).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gotb, wantb)
    assert differ > 0, "no element separates one rounding from a level-by-level fp32 sum"


def pin_code_range(o):
    """Codes index codewords 0 .. K-1 (a code is a codeword number): the largest valid code
    K-1 is accepted and decodes to codeword K-1; a code equal to K is refused by the code
    check and by every operation that reads codes."""
    K = 5
    cb = np.arange(2 * 3 * K * 2, dtype=np.float32).reshape(2, 3, K, 2)
    codes = np.full((4, 2, 3), K - 1, np.uint16)
    assert o.check_codes(codes, K) == 0
    out, _ = o.decode_rows(codes, cb, False, np.array([2], np.int32), False)
    assert np.array_equal(out[0], cb[0, :, K - 1].reshape(-1) + cb[1, :, K - 1].reshape(-1))
    bad = codes.copy()
    bad[3, 1, 2] = K
    assert o.check_codes(bad, K) != 0
    for call in (lambda: o.decode_rows(bad, cb, False, np.array([3], np.int32), False),
                 lambda: o.matvec(bad, cb, False, np.ones((1, 6))),
                 lambda: o.logits(bad, cb, False, np.ones((1, 6), np.float32), 30.0)):
        try:
            call()
        except ValueError:
            continue
        raise AssertionError("a code equal to K was accepted")


def pin_bf16_rounding(o):
    """Round-to-nearest-even ties on hand-checked values (1 + 2^-8 -> 1; 1 + 3*2^-8 -> 1 + 2^-6)."""
    cb = np.zeros((1, 1, 4, 1), np.float32)
    cb[0, 0, :, 0] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8 + 2.0 ** -20), 3.0]
    codes = np.arange(4, dtype=np.uint16).reshape(4, 1, 1)
    out, _ = o.decode_rows(codes, cb, False, np.arange(4), True)
    got = synth.bf16_bits_to_f32(out[:, 0])
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, -(1.0 + 2.0 ** -7), 3.0]


# --------------------------------------------------------------------------- LUT build

def pin_build_lut_scalar_subspaces(o):
    """d=1: LUT[b][l][m][k] = x[b][m] * C[l][m][k][0] (numpy outer product); bf16 codebooks widened exactly."""
    rng = np.random.default_rng(17)
    cb = rng.normal(0, 0.02, size=(2, 5, 7, 1)).astype(np.float32)
    x = rng.standard_normal((3, 5))
    lut = o.build_lut(cb, False, x)
    ref = x[:, None, :, None] * cb[None, :, :, :, 0].astype(np.float64)
    assert np.array_equal(lut, ref)
    bits = synth.f32_to_bf16_bits(cb)
    lutb = o.build_lut(bits, True, x)
    refb = x[:, None, :, None] * synth.bf16_bits_to_f32(bits)[None, :, :, :, 0].astype(np.float64)
    assert np.array_equal(lutb, refb)


def pin_build_lut_dot(o):
    """d>1: each table entry is the dot product of one subvector of x with one codeword (numpy einsum)."""
    rng = np.random.default_rng(18)
    L, M, K, d = 2, 3, 4, 5
    cb = rng.normal(0, 0.02, size=(L, M, K, d)).astype(np.float32)
    x = rng.standard_normal((2, M * d))
    lut = o.build_lut(cb, False, x)
    ref = np.einsum("bmj,lmkj->blmk", x.reshape(2, M, d), cb.astype(np.float64))
    assert _rel(lut, ref) <= 1e-14


# --------------------------------------------------------------------------- MLP

def pin_matvec_identity_codebook(o):
    """M=1, d=D, L=1, K=rows, code[r]=r: the coded matrix is the codebook itself; y = numpy matmul."""
    rng = np.random.default_rng(19)
    rows, D = 40, 24
    cb = rng.normal(0, 0.02, size=(1, 1, rows, D)).astype(np.float32)
    codes = np.arange(rows, dtype=np.uint16).reshape(rows, 1, 1)
    x = rng.standard_normal((2, D))
    y = o.matvec(codes, cb, False, x)
    assert _rel(y, x @ cb[0, 0].astype(np.float64).T) <= 1e-13


def pin_gelu_tanh(o):
    """gelu_tanh against torch's GELU(approximate='tanh') and within the tanh approximation's
    known distance (< 5e-4) of the exact erf GELU; gelu_mul multiplies by the up projection."""
    t = np.linspace(-9.0, 9.0, 721)
    got = o.gelu_tanh(t)
    ref = torch.nn.functional.gelu(torch.from_numpy(t), approximate="tanh").numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-14)
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in t])
    assert np.abs(got - exact).max() < 5e-4
    assert o.gelu_tanh(0.0) == 0.0
    u = np.linspace(-2, 2, 721)
    assert np.allclose(o.gelu_mul(t, u), ref * u, rtol=0, atol=1e-14)


def pin_mlp_chain(o):
    """y = W_down (gelu_tanh(W_gate x) * W_up x), checked against dense numpy on decoded weights."""
    rng = np.random.default_rng(20)
    hid, inter = 8, 12
    gate = synth.gen_matrix(rng, inter, hid, 4, 5, 2, (0.02, 0.005), "f32")
    up = synth.gen_matrix(rng, inter, hid, 4, 5, 2, (0.02, 0.005), "f32")
    down = synth.gen_matrix(rng, hid, inter, 6, 5, 2, (0.02, 0.005), "f32")
    x = rng.standard_normal((1, hid)).astype(np.float32)

    def dense(m):   # fp64 gather of the codewords with numpy fancy indexing
        W = np.zeros((m.rows, m.M, m.d))
        for l in range(m.L):
            W += m.codebooks[l, np.arange(m.M)[None, :], m.codes[:, l, :].astype(np.int64)]
        return W.reshape(m.rows, m.D)

    g, u, a, y = o.mlp((gate.codes, gate.codebooks, False), (up.codes, up.codebooks, False),
                       (down.codes, down.codebooks, False), x)
    gd = x.astype(np.float64) @ dense(gate).T
    ud = x.astype(np.float64) @ dense(up).T
    ad = torch.nn.functional.gelu(torch.from_numpy(gd), approximate="tanh").numpy() * ud
    yd = ad @ dense(down).T
    assert _rel(g, gd) <= 1e-12 and _rel(u, ud) <= 1e-12 and _rel(y, yd) <= 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
