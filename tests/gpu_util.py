"""Shared helpers of the GPU parity tests: device upload and the comparison rules.

Comparison rules (the tolerances the tests enforce):
  - integer and byte work (packed codes, decoded rows, ids) is compared bit for bit;
  - fp32-table logits: |gpu - oracle| <= 1e-5 * max|oracle| for each batch entry;
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
