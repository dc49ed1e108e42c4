"""Shared helpers of the GPU parity tests: device upload and the comparison rules.

Comparison rules (the tolerances the tests enforce):
  - integer and byte work (packed codes, decoded rows, ids) is compared bit for bit;
  - fp32-table logits: |gpu - oracle| <= 1e-5 * max|oracle| for each batch entry, all values finite;
  - bf16-table logits: per element 2^-8 * sum_{l,m} |LUT64 entry used| + 1e-5 * max|oracle|
    (twice the bf16 rounding bound of every looked-up entry; the softcap's slope <= 1 keeps it);
  - argmax: the GPU id is the lowest index of the maximum of the GPU's own logits, and its oracle
    logit is within 2*tol of the oracle maximum (ties within tolerance admit several answers).
"""
import numpy as np
import torch

import lut_logits_amd as la
import oracle

REL_TOL = 1e-5


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def oracle_head(mat, h, softcap):
    return oracle.default().logits(mat.codes, mat.codebooks, mat.cb_is_bf16, h, softcap)


def check_logits(gpu, ref, tol=None):
    """Per batch entry: max |gpu - ref| <= tol (default 1e-5 * max|ref|). Returns the worst relative error."""
    gpu = np.asarray(gpu, np.float64)
    assert np.isfinite(ref).all(), "the oracle's values are not all finite"
    assert np.isfinite(gpu).all(), f"{int((~np.isfinite(gpu)).sum())} GPU values are not finite"
    worst = 0.0
    for b in range(ref.shape[0]):
        scale = max(np.abs(ref[b]).max(), 1e-30)
        t = REL_TOL * scale if tol is None else tol[b]
        err = np.abs(gpu[b] - ref[b])
        bad = np.nonzero(err > t)[0]
        assert bad.size == 0, f"b={b}: {bad.size} logits out of tolerance, first at {bad[0]}: gpu {gpu[b, bad[0]]} ref {ref[b, bad[0]]}"
        worst = max(worst, float(err.max() / scale))
    return worst


def check_argmax(am_gpu, logits_gpu, ref, tol=None):
    for b in range(ref.shape[0]):
        row = logits_gpu[b]
        assert am_gpu[b] == int(np.argmax(row)), f"b={b}: argmax {am_gpu[b]} is not the first maximum of the GPU logits"
        t = REL_TOL * np.abs(ref[b]).max() if tol is None else tol[b]
        assert ref[b, am_gpu[b]] >= ref[b].max() - 2 * t, f"b={b}: argmax {am_gpu[b]} is not a maximum of the oracle"


def to_dev(mat, layout="blocked"):
    return la.to_device(mat, layout=layout)


def bf16_table_tol(mat, h, ref, chunk=8):
    """Per-element tolerance of logits from a bf16 table: 2^-8 * sum_{l,m} |LUT64 entry used| + 1e-5 * max|ref|
    (twice the RNE unit roundoff of every looked-up entry), built a few vectors at a time."""
    o = oracle.default()
    tol = np.empty_like(ref)
    for b0 in range(0, h.shape[0], chunk):
        lut64 = o.build_lut(mat.codebooks, mat.cb_is_bf16, h[b0:b0 + chunk])
        tol[b0:b0 + chunk] = 2.0 ** -8 * o.lut_sum(mat.codes, np.abs(lut64))
    return tol + REL_TOL * np.abs(ref).max(axis=1, keepdims=True)


def check_topk(g, ids, vals, am, ref, tolv, k):
    """Top-k rules: self-consistency with the GPU's own logits (value desc, id asc), the oracle's
    must-include set, every id within 2t of the oracle's k-th value, and exact ids at every rank whose
    gaps to both neighbours exceed 2t (t = the worst per-element tolerance of that vector)."""
    for b in range(ref.shape[0]):
        order = np.lexsort((np.arange(g.shape[1]), -g[b]))[:k]
        assert np.array_equal(ids[b], order), f"b={b}: top-k is not that of the GPU logits"
        assert np.array_equal(vals[b], g[b, order])
        if am is not None:
            assert am[b] == ids[b, 0]
        t = tolv[b].max()
        kth = np.sort(ref[b])[::-1][k - 1]
        must = np.nonzero(ref[b] > kth + 2 * t)[0]
        assert set(must.tolist()) <= set(ids[b].tolist()), f"b={b}: an oracle top-k id is missing"
        assert np.all(ref[b, ids[b]] >= kth - 2 * t), f"b={b}: a returned id is below the oracle's k-th"
        oref = np.lexsort((np.arange(ref.shape[1]), -ref[b]))[:k]
        srt = ref[b, oref]
        for i in range(k):
            lo = srt[i + 1] if i + 1 < k else kth - 1e9
            hi = srt[i - 1] if i > 0 else srt[i] + 1e9
            if hi - srt[i] > 2 * t and srt[i] - lo > 2 * t:
                assert ids[b, i] == oref[i], f"b={b}: rank {i} differs where the gaps exceed 2t"
