"""Byte and multiply-add ledgers for factored projections.

Pure arithmetic used by the benchmark to turn kernel times into algorithmic
GB/s and TFLOP/s, and by the tests to reproduce the pages' worked numbers.
Page cited: "DictLLM: Shared Dictionaries for Post-Training Compression"
(technical review), sections "The budget: trading shared rank against
sparsity" (Eq. (2), (3)) and "From retained values to measured decoding"
(NVFP4 accounting, Eq. (12), the multiply-add model).
"""
from __future__ import annotations

import math

# ------------------------------------------------------------ pages' formulas


def group_values(n: int, d_in: int, d_out: int, k: int, p: float) -> float:
    """Eq. (2): N_p = d_in*k + n*(1-p)*k*d_out retained values of a group."""
    return d_in * k + n * (1.0 - p) * k * d_out


def dense_values(n: int, d_in: int, d_out: int) -> int:
    """Eq. (2): N_0 = n*d_in*d_out."""
    return n * d_in * d_out


def rank_for_budget(rho_fac: float, n: int, d_in: int, d_out: int) -> int:
    """Eq. (3): k = floor((1 - rho_fac) n d_in d_out / (d_in + n d_out))."""
    return math.floor((1.0 - rho_fac) * n * d_in * d_out / (d_in + n * d_out))


def sparse_saves_bytes_threshold(a: float, b: float, h: float) -> float:
    """Eq. (12): sparse storage (a index bits per kept value, h overhead bits
    per logical position, b bits per value) beats dense iff p > (a+h)/(b+a)."""
    return (a + h) / (b + a)


def nvfp4_bits_per_value() -> float:
    """4-bit value plus an 8-bit scale shared by 16 values."""
    return 4.0 + 8.0 / 16.0


VALUE_BITS = {"f16": 16.0, "fp8": 8.0, "int8": 8.0}


def value_bits(fmt: str) -> float:
    """Bits per retained value under the values-only accounting of the
    pages (outer scales, indices and padding left out)."""
    return nvfp4_bits_per_value() if fmt == "nvfp4" else VALUE_BITS[fmt]


def mixed_gain(dict_share: float, dfmt: str, cfmt: str) -> float:
    """Storage gain over an all-FP16 factorised model whose retained values
    are a fraction ``dict_share`` in D and the rest in C (tables page,
    Table 4: the gain of each factor-format pair)."""
    bits = dict_share * value_bits(dfmt) + (1.0 - dict_share) * value_bits(cfmt)
    return 16.0 / bits


def dict_share_from_gain(gain: float, dfmt: str, cfmt: str) -> float:
    """Inverse of ``mixed_gain`` in ``dict_share``."""
    bd, bc = value_bits(dfmt), value_bits(cfmt)
    return (16.0 / gain - bc) / (bd - bc)


def macs_factored(n: int, k: int, d_in: int, d_out: int, p: float) -> float:
    """Per group and token: n*k*(d_in + (1-p)*d_out) multiply-adds."""
    return n * k * (d_in + (1.0 - p) * d_out)


def macs_dense(n: int, d_in: int, d_out: int) -> int:
    return n * d_in * d_out


# ------------------------------------------------------------ storage bytes

ELEM_BYTES = {"f32": 4.0, "f16": 2.0}


def nvfp4_bytes(n_elems: int) -> int:
    """codes ceil(n/2) + one scale byte per 16 elements + 4-byte tensor scale."""
    return (n_elems + 1) // 2 + (n_elems + 15) // 16 + 4


def dict_bytes(d_in: int, k: int, dtype: str) -> int:
    if dtype == "nvfp4":
        return nvfp4_bytes(d_in * k)
    return int(d_in * k * ELEM_BYTES[dtype])


def csc_bytes(d_out: int, nnz: int, dtype: str) -> int:
    """colptr int32[d_out+1] + uint16 row indices + values (8-bit codes:
    one byte per entry plus one fp32 scale per column)."""
    base = 4 * (d_out + 1) + 2 * nnz
    if dtype == "nvfp4":
        return base + nvfp4_bytes(nnz)
    if dtype in ("fp8", "int8"):
        return base + nnz + 4 * d_out
    return base + int(nnz * ELEM_BYTES[dtype])


def bcsc_bytes(d_out: int, nblk: int, dtype: str) -> int:
    """Block-structured coefficients, blocks of 8 consecutive atoms:
    colptr int32[d_out+1] + one uint16 block index and 8 values per kept
    block."""
    return 4 * (d_out + 1) + nblk * (2 + int(8 * ELEM_BYTES[dtype]))


def bcsc_density_at_equal_bytes(k: int, d_out: int, nnz: int, dtype: str) -> float:
    """Fraction of blocks a block-structured C may keep for the bytes of an
    unstructured CSC with nnz entries in the same dtype (the equal packed
    bytes comparison of the Review, "Let the accelerator constrain the
    support")."""
    per_block = 2 + 8 * ELEM_BYTES[dtype]
    nblk = (csc_bytes(d_out, nnz, dtype) - 4 * (d_out + 1)) / per_block
    return nblk / (((k + 7) // 8) * d_out)


def act_bytes(T: int, width: int, dtype: str) -> int:
    return int(T * width * ELEM_BYTES[dtype])


def group_bytes(*, d_in: int, d_out: int, k: int, T: int, nnzs, wdtype: str, cdtype: str,
                xdtype: str, ydtype: str) -> int:
    """Algorithmic bytes of one group forward: the dictionary once, and per
    layer its coefficients, its activations and its outputs.  The intermediate
    Z is not counted."""
    total = dict_bytes(d_in, k, wdtype)
    for nnz in nnzs:
        total += csc_bytes(d_out, nnz, cdtype) + act_bytes(T, d_in, xdtype) + act_bytes(
            T, d_out, ydtype)
    return total


def group_flops(*, d_in: int, k: int, T: int, nnzs) -> tuple[int, int]:
    """(dense X.D flops, sparse Z.C useful flops) of one group forward."""
    n = len(nnzs)
    return 2 * n * T * d_in * k, 2 * T * int(sum(nnzs))
