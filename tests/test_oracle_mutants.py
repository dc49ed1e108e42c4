"""Plausible mistakes planted in copies of the oracle must each fail at least one pin.

Each mutant is a one-place textual change to oracle/rq_oracle.c (a dropped
term, a transposed index, a wrong sign or constant, a wrong tie-break),
compiled on the CPU into a temporary library. The shipped oracle is never
modified. All mutants keep every memory access in bounds.
"""
import os

import pytest

import oracle
from oracle.build import SRC, build
from oracle_pins import ALL_PINS

MUTANTS = {
    "drop_last_level": (
        "s += codebook_value(cb, cb_is_bf16, cb_pos(l, m, k, j, M, K, d));",
        "if (l + 1 < L || L == 1) s += codebook_value(cb, cb_is_bf16, cb_pos(l, m, k, j, M, K, d));"),
    "codes_layout_m_major": (
        "return ((size_t)r * L + l) * (size_t)M + m;",
        "return ((size_t)r * M + m) * (size_t)L + l;"),
    "codebook_k_j_transposed": (
        "return (((size_t)l * M + m) * (size_t)K + k) * (size_t)d + j;",
        "return (((size_t)l * M + m) * (size_t)d + j) * (size_t)K + k;"),
    "subspace_offset_transposed": (
        "w[(size_t)m * d + j] = s;",
        "w[(size_t)j * M + m] = s;"),
    "dot_skips_last_dim": (
        "for (int i = 0; i < D; ++i) acc += w[i] * xb[i];",
        "for (int i = 0; i + 1 < D; ++i) acc += w[i] * xb[i];"),
    "softcap_missing_scale": (
        "return c * tanh(z / c);",
        "return tanh(z / c);"),
    "softcap_inverted_argument": (
        "return c * tanh(z / c);",
        "return c * tanh(z * c);"),
    "argmax_last_of_ties": (
        "if (row[v] > row[best]) best = v;",
        "if (row[v] >= row[best]) best = v;"),
    "topk_ties_by_id_descending": (
        "return (a->id < b->id) ? -1 : (a->id > b->id);",
        "return (a->id > b->id) ? -1 : (a->id < b->id);"),
    "bf16_truncates": (
        "return (uint16_t)((u + 0x7fffu + lsb) >> 16);",
        "return (uint16_t)((u + 0u * lsb) >> 16);"),
    "gelu_wrong_cubic_coefficient": (
        "0.044715 * t * t * t",
        "0.04715 * t * t * t"),
    "gelu_missing_half": (
        "return 0.5 * t * (1.0 + tanh(",
        "return t * (1.0 + tanh("),
    "lut_build_wrong_subvector": (
        "s += x[(size_t)b * D + (size_t)m * d + j]",
        "s += x[(size_t)b * D + (size_t)m + j]"),
    "lut_sum_level0_only": (
        "acc += lut[(((size_t)b * L + l) * M + m) * (size_t)K + k];",
        "acc += lut[(((size_t)b * L + 0) * M + m) * (size_t)K + k];"),
    "decode_levels_summed_in_fp32": (
        "s += codebook_value(cb, cb_is_bf16, cb_pos(l, m, k, j, M, K, d));",
        "s = (float)(s + codebook_value(cb, cb_is_bf16, cb_pos(l, m, k, j, M, K, d)));"),
    "code_check_admits_k": (
        "if (codes[i] >= K) return OR_ERR_CODE;",
        "if (codes[i] > K) return OR_ERR_CODE;"),
    "decode_code_check_admits_k": (
        "if (codes[code_pos(r, l, m, L, M)] >= K) { free(w); return OR_ERR_CODE; }",
        "if (codes[code_pos(r, l, m, L, M)] > K) { free(w); return OR_ERR_CODE; }"),
    "lut_sum_first_code_of_row": (
        "int k = codes[code_pos(r, l, m, L, M)];\n          acc +=",
        "int k = codes[code_pos(r, l, 0, L, M)];\n          acc +="),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = build(src=path, out=os.path.join(tmp_path, f"lib_{name}.so"), extra=["-w"])
    o = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError) as e:   # ValueError: the oracle refused its input
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"no pin catches mutant {name}"
