"""Storage and residency accounting for RQ-coded matrices (host logic).

The Gemma-2-2B pages quote sizes for the coded embedding and MLP matrices;
these closed forms reproduce them and size the buffers the library reads:
  - codes: rows * L * M codes, stored 16-bit in memory (runtime-compression
    page, memory paragraph: "codes as int16") or bit-packed at log2(K) bits
    for the on-disk artifact (1,180 MB -> 265 MB, opening paragraph);
  - codebooks: one K x d table per (level, subspace), fp32 on the pages;
  - the dense reference is rows * D bf16 values.
"""
import math

MB = 1e6


def dense_bytes(rows, D, bits=16):
    return rows * D * bits // 8


def code_bytes(rows, L, M, bits=16):
    """Bytes of rows*L*M codes at `bits` bits each (16: the in-memory int16 layout)."""
    return (rows * L * M * bits + 7) // 8


def codebook_bytes(L, M, K, d, bits=32):
    return L * M * K * d * bits // 8


def packed_code_bits(K):
    return max(1, math.ceil(math.log2(K)))


def artifact_bytes(rows, D, M, K, L, cb_bits=32, packed=False):
    """Codes (16-bit, or packed at log2 K bits) plus codebooks."""
    d = D // M
    bits = packed_code_bits(K) if packed else 16
    return code_bytes(rows, L, M, bits) + codebook_bytes(L, M, K, d, cb_bits)


def bits_per_param(rows, D, M, K, L, cb_bits=32, packed=True):
    return artifact_bytes(rows, D, M, K, L, cb_bits, packed) * 8 / (rows * D)


def lut_bytes(B, L, M, K, bits=32):
    return B * L * M * K * bits // 8


def mlp_average_bpp(hidden, inter, d, K_gate_up, K_down, L, cb_bits=32):
    """Average bits/param over gate, up (inter x hidden) and down (hidden x inter); the three
    matrices hold equally many parameters, so the plain mean is the parameter-weighted mean."""
    g = bits_per_param(inter, hidden, hidden // d, K_gate_up, L, cb_bits)
    dn = bits_per_param(hidden, inter, inter // d, K_down, L, cb_bits)
    return (2 * g + dn) / 3
