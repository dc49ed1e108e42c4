"""Storage-format closed forms against the numbers the pages print (tests/golden/page_numbers.json)."""
import json
import os

import pytest

from lut_logits_amd import formats as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))
V, D, M, K, L = 256000, 2304, 384, 1024, 2   # runtime-compression page, LUT-serving paragraph
d = D // M


def near(key, got):
    g = GOLD[key]
    assert abs(got - g["value"]) <= g["tol"], (key, got, g)


def test_embedding_sizes():
    near("embedding_params", V * D)
    near("embedding_bf16_MB", F.dense_bytes(V, D) / F.MB)
    near("rq_resident_MB", F.artifact_bytes(V, D, M, K, L, cb_bits=32, packed=False) / F.MB)
    near("rq_storage_MB", F.artifact_bytes(V, D, M, K, L, cb_bits=32, packed=True) / F.MB)
    near("rq_bits_per_param", F.bits_per_param(V, D, M, K, L, cb_bits=32, packed=True))
    near("lut_idle_saving_MB", (F.dense_bytes(V, D) - F.artifact_bytes(V, D, M, K, L, 32, False)) / F.MB)


def test_one_shared_codebook_would_not_match():
    """Codebooks are per (level, subspace): a single K x d table per level gives 393 MB, not 412 MB."""
    shared = F.code_bytes(V, L, M) + L * K * d * 4
    assert abs(shared / F.MB - GOLD["rq_resident_MB"]["value"]) > 10


def test_mlp_bits_per_param():
    hidden, inter = 2304, 9216
    near("mlp_params", 26 * 3 * hidden * inter)
    near("mlp_first_attempt_bpp", F.mlp_average_bpp(hidden, inter, d=8, K_gate_up=1024, K_down=1024, L=2))
    near("mlp_v2_bpp", F.mlp_average_bpp(hidden, inter, d=8, K_gate_up=1024, K_down=256, L=2))


def test_lut_and_code_sizes():
    assert F.code_bytes(V, L, M) == 393_216_000
    assert F.lut_bytes(1, L, M, K) == 3_145_728
    assert F.codebook_bytes(L, M, K, d, 16) == 9_437_184
    assert F.packed_code_bits(1024) == 10 and F.packed_code_bits(256) == 8 and F.packed_code_bits(1) == 1


@pytest.mark.parametrize("K_", [1, 2, 255, 256, 257, 4096])
def test_packed_bits_cover_all_codes(K_):
    assert 2 ** F.packed_code_bits(K_) >= K_
