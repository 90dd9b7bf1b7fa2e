"""Pins of the oracle's 8-bit coefficient codes (CPU only).

Table 4 of the tables page ("DictLLM: Post-training Compression of Large
Language Model with Dictionary Kernels") pairs an NVFP4 dictionary with FP8
or INT8 coefficients.  The pages leave the scaling of those codes open; the
oracle reads it as one fp32 scale per column, amax / 448 (E4M3) or amax / 127
(INT8), nearest code with ties to even.  What fixes the oracle, other than
itself:
  * INT8 rounding: hand-checked ties and clamps (round half to even is the
    definition), and numpy's rint over random values;
  * E4M3 codes: torch's float8_e4m3fn conversion of the same fp32 quotient;
  * per-column properties: the largest magnitude of a column takes the top
    code, zero columns take scale 1, the round-trip error stays within half
    a code step times the scale;
  * the forward with 8-bit C equals numpy's dense product with C decoded
    independently (torch's E4M3 table, two's-complement bytes).
"""
import numpy as np
import pytest
import torch

import oracle as O
from test_oracle_forward import _decode_nvfp4_numpy


def test_int8_nearest_ties_and_clamp():
    # exact quotients (scale 1): halves go to the even neighbour
    cases = {127.0: 127, 63.5: 64, 62.5: 62, -62.5: -62, -63.5: -64, 2.5: 2, 3.5: 4,
             -0.5: 0, 0.5: 0, 1.5: 2, 0.49: 0, -0.51: -1, 126.5: 126, 127.4: 127,
             200.0: 127, -1e9: -127, -127.6: -127}
    for v, want in cases.items():
        assert O.int8_nearest(v) == want, v


def test_int8_nearest_matches_numpy_rint():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-130, 130, 5000).astype(np.float32),
                        (np.arange(-255, 256) / np.float32(2)).astype(np.float32)])
    want = np.clip(np.rint(v), -127, 127).astype(int)
    got = np.array([O.int8_nearest(x) for x in v])
    assert np.array_equal(got, want)


def _csc(rng, k, d_out, density, dtype=np.float16, scale_cols=True):
    Cd = rng.standard_normal((k, d_out)) * (rng.random((k, d_out)) < density)
    if scale_cols:  # columns over several orders of magnitude
        Cd = Cd * np.exp(rng.uniform(-6, 3, d_out))[None, :]
    return O.pack_csc(Cd.astype(dtype))


def _col_of_entries(c):
    return np.repeat(np.arange(c.d_out), np.diff(c.colptr))


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_fp8_codes_match_torch_e4m3(dtype):
    rng = np.random.default_rng(11)
    c = _csc(rng, 96, 70, 0.3, dtype)
    q = O.quantize8_csc(c, "fp8").vals
    v = np.asarray(c.vals, np.float32)
    col = _col_of_entries(c)
    amax = np.zeros(c.d_out, np.float32)
    np.maximum.at(amax, col, np.abs(v))
    s = amax / np.float32(448.0)
    s[s == 0] = 1.0
    assert np.array_equal(q.col_scale, s)
    quot = v / s[col]                      # fp32, one rounding each
    want = torch.tensor(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q.codes, want)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_int8_codes_match_numpy(dtype):
    rng = np.random.default_rng(12)
    c = _csc(rng, 96, 70, 0.3, dtype)
    q = O.quantize8_csc(c, "int8").vals
    v = np.asarray(c.vals, np.float32)
    col = _col_of_entries(c)
    amax = np.zeros(c.d_out, np.float32)
    np.maximum.at(amax, col, np.abs(v))
    s = amax / np.float32(127.0)
    s[s == 0] = 1.0
    assert np.array_equal(q.col_scale, s)
    want = np.clip(np.rint(v / s[col]), -127, 127).astype(np.int8).view(np.uint8)
    assert np.array_equal(q.codes, want)


def _decode(q, col):
    if q.kind == "fp8":
        val = torch.tensor(q.codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        val = q.codes.view(np.int8).astype(np.float64)
    return val * q.col_scale[col].astype(np.float64)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_round_trip_error_and_top_code(kind):
    rng = np.random.default_rng(13)
    c = _csc(rng, 128, 90, 0.25, np.float32)
    q = O.quantize8_csc(c, kind).vals
    col = _col_of_entries(c)
    v = np.asarray(c.vals, np.float64)
    dec = _decode(q, col)
    s = q.col_scale[col].astype(np.float64)
    if kind == "int8":
        # half a unit of the integer grid, plus the fp32 rounding of v / s
        assert np.all(np.abs(dec - v) <= s * (0.5 + 1e-5))
    else:
        # E4M3: half a step at the value's binade (3 mantissa bits), and
        # half of the subnormal step 2^-9 below 2^-6
        a = np.abs(v / s)
        step = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 3),
                        2.0 ** -9)
        assert np.all(np.abs(dec - v) <= s * (0.5 * step * (1 + 1e-5) + 1e-12))
    # each non-empty column's largest magnitude takes the top code
    top = 0x7E if kind == "fp8" else 127
    for j in range(c.d_out):
        lo, hi = c.colptr[j], c.colptr[j + 1]
        if hi > lo:
            i = lo + np.argmax(np.abs(v[lo:hi]))
            mag = q.codes[i] & 0x7F if kind == "fp8" else abs(int(q.codes[i:i + 1].view(np.int8)[0]))
            assert mag == top, j


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_zero_column_negative_zero_and_signs(kind):
    Cd = np.zeros((8, 3), np.float32)
    Cd[1, 0], Cd[5, 0] = -2.0, 0.5        # column 0: amax 2
    Cd[2, 2] = 3.0                        # column 1 stays empty
    c = O.pack_csc(Cd)
    q = O.quantize8_csc(c, kind).vals
    qmax = 448.0 if kind == "fp8" else 127.0
    assert q.col_scale[1] == 1.0
    assert q.col_scale[0] == np.float32(2.0) / np.float32(qmax)
    dec = _decode(q, _col_of_entries(c))
    assert abs(dec[0] + 2.0) < 1e-6       # the column maximum comes back
    assert np.sign(dec[0]) == -1 and np.sign(dec[2]) == 1
    # a column of zeros in a CSC is impossible (the packer drops them), but
    # quantising tiny values gives exact zero codes of the right kind
    tiny = O.CSC(4, 1, np.array([0, 2], np.int32), np.array([0, 3], np.uint16),
                 np.array([1.0, -1e-30], np.float32))
    qt = O.quantize8_csc(tiny, kind).vals
    if kind == "fp8":
        assert qt.codes[1] == 0x80        # -0 keeps its sign bit
    else:
        assert qt.codes[1] == 0


def test_quantize8_rejects_non_finite():
    for bad in (np.nan, np.inf, -np.inf):
        c = O.CSC(4, 1, np.array([0, 2], np.int32), np.array([0, 3], np.uint16),
                  np.array([1.0, bad], np.float32))
        for kind in ("fp8", "int8"):
            with pytest.raises(ValueError):
                O.quantize8_csc(c, kind)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("nvfp4_dict", [False, True])
def test_forward_with_8bit_codes_matches_dense_product(kind, nvfp4_dict):
    rng = np.random.default_rng(14)
    T, d_in, k, d_out = 3, 64, 48, 40
    X = rng.standard_normal((T, d_in)).astype(np.float16)
    Dt = (rng.standard_normal((k, d_in)) / 8).astype(np.float32)   # atom-major
    c = O.quantize8_csc(_csc(rng, k, d_out, 0.35, np.float16), kind)
    if nvfp4_dict:
        D = O.nvfp4_pack(Dt)
        Dv = _decode_nvfp4_numpy(D).reshape(k, d_in)
    else:
        D, Dv = Dt, Dt.astype(np.float64)
    Y = O.forward(X, D, d_in, c)
    Cdense = np.zeros((k, d_out))
    Cdense[c.rowidx.astype(int), _col_of_entries(c)] = _decode(c.vals, _col_of_entries(c))
    ref = X.astype(np.float64) @ Dv.T @ Cdense
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)
