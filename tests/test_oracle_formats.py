"""Pins of the oracle's NVFP4 codecs (CPU only).

What fixes them, other than the oracle itself:
  * E2M1 values: the OCP MX element table (tests/golden/e2m1_values.txt).
  * E4M3 values and rounding: torch's float8_e4m3fn conversions (a library
    routine), over every code and over values that include every midpoint.
  * The quantiser: brute-force nearest-grid search in numpy, the round trip of
    all 16 E2M1 codes, an error bound, and the 4.5-bit accounting of the
    technical review ("From retained values to measured decoding").
"""
import numpy as np
import pytest
import torch

import oracle as O


def test_e2m1_values_match_ocp_table(golden):
    for code, val in golden("e2m1_values.txt"):
        code, val = int(code), float(val)
        assert O.e2m1_value(code) == val
        assert O.e2m1_value(code | 8) == -val
        assert np.signbit(O.e2m1_value(code | 8))


def test_e4m3_values_match_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got = O.e4m3_value(c)
        if np.isnan(ref[c].item()):
            assert np.isnan(got), c
        else:
            assert got == ref[c].item(), c


def _torch_e4m3(vals):
    t = torch.tensor(np.asarray(vals, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_nearest_matches_torch_rne():
    # every finite positive code, every midpoint between neighbours, and
    # random fp32 values spread over the range (torch rounds to nearest even
    # and overflows to NaN above 464, so stay at or below 464)
    vals = [O.e4m3_value(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    rng = np.random.default_rng(7)
    rnd = np.exp(rng.uniform(np.log(1e-5), np.log(464.0), 20000)).astype(np.float32)
    tests = np.concatenate([np.float32(vals), np.float32(mids), rnd, np.float32([464.0, 0.0])])
    ref = _torch_e4m3(tests)
    got = np.array([O.e4m3_nearest(v) for v in tests])
    assert np.array_equal(got, ref)


def test_e4m3_nearest_saturates():
    for v in (448.0, 464.0, 465.0, 1e6, 3.0e38):
        assert O.e4m3_nearest(v) == 0x7E


def test_e2m1_nearest_is_nearest_with_even_ties():
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(3)
    vs = np.concatenate([grid, mids, -mids, rng.uniform(-8, 8, 5000), [7.0, 100.0, -0.0]])
    for v in vs.astype(np.float32):
        c = O.e2m1_nearest(v)
        d = np.abs(np.abs(v) - grid)
        assert d[c] == d.min(), (v, c)
        ties = np.flatnonzero(d == d.min())
        if ties.size > 1:
            assert c % 2 == 0 and c in ties, (v, c)


def _brute_nvfp4(x):
    """numpy restatement of the quantiser by brute force on the value grid
    (independent of the oracle's nearest-code searches): for each block pick
    the scale by torch's e4m3 cast, then each element the grid point
    m*s*ts nearest to x in fp32 division terms."""
    x = np.asarray(x, np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    ts = np.float32(amax / np.float32(2688.0))
    if ts == 0:
        ts = np.float32(1.0)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    codes = np.zeros(x.size, np.int64)
    scales = []
    for b in range(0, x.size, 16):
        blk = x[b:b + 16]
        bmax = np.float32(np.abs(blk).max())
        sf = np.float32(bmax / np.float32(np.float32(6.0) * ts))
        sc = int(_torch_e4m3([min(sf, np.float32(448.0))])[0])
        s = np.float32(torch.tensor([sc], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item())
        denom = np.float32(s * ts)
        scales.append(sc)
        for i, xi in enumerate(blk):
            if denom == 0:
                mag = 0
            else:
                v = abs(float(np.float32(xi / denom)))
                d = np.abs(v - grid)
                cand = np.flatnonzero(d == d.min())
                mag = int(cand[0]) if cand.size == 1 else int([c for c in cand if c % 2 == 0][0])
            codes[b + i] = mag | (8 if np.signbit(xi) else 0)
    return codes, np.array(scales, np.int64), ts


def _codes_of(q):
    lo = q.codes & 15
    hi = q.codes >> 4
    return np.stack([lo, hi], 1).reshape(-1)[: q.n].astype(np.int64)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 64, 333])
def test_nvfp4_pack_matches_brute_force(n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.exp(rng.uniform(-3, 3, n))).astype(np.float32)
    x[::7] = 0.0
    if n > 3:
        x[3] = -0.0
    q = O.nvfp4_pack(x)
    codes, scales, ts = _brute_nvfp4(x)
    assert q.ts == ts
    assert np.array_equal(q.scales.astype(np.int64), scales)
    assert np.array_equal(_codes_of(q), codes)


def test_nvfp4_round_trip_all_16_codes():
    # a block holding each E2M1 value once (and its negatives in the next
    # block) with a tensor whose amax is 6: ts = 6/2688, every block's scale
    # is 448, so denom = 448 * ts = 1 up to one fp32 rounding and every code
    # must come back unchanged.
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    x = np.concatenate([grid, grid, -grid, -grid]).astype(np.float32)
    q = O.nvfp4_pack(x)
    codes = _codes_of(q)
    want = np.concatenate([np.arange(8), np.arange(8), np.arange(8) | 8, np.arange(8) | 8])
    assert np.array_equal(codes, want)
    assert np.all(q.scales == 0x7E)
    y = O.nvfp4_unpack(q)
    # each value comes back within one fp32 ulp (through ts)
    assert np.all(np.abs(y - x) <= np.spacing(np.abs(x).astype(np.float32)) + 0)
    assert np.array_equal(np.signbit(y), np.signbit(x))


def test_nvfp4_error_bound_and_scale_of_amax_block():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(4096).astype(np.float32)
    q = O.nvfp4_pack(x)
    y = O.nvfp4_unpack(q).astype(np.float64)
    # the block holding amax gets the largest scale code and a +-6 code there
    i = int(np.argmax(np.abs(x)))
    assert q.scales[i // 16] == 0x7E
    assert (_codes_of(q)[i] & 7) == 7
    # |x - xhat| <= half the local grid gap times s*ts (plus fp32 rounding)
    gaps = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])
    codes = _codes_of(q)
    for b in range(0, x.size, 16):
        s = O.e4m3_value(int(q.scales[b // 16])) * q.ts
        for j in range(b, b + 16):
            bound = gaps[codes[j] & 7] / 2 * s
            assert abs(x[j] - y[j]) <= bound * (1 + 1e-6) + 1e-30


def test_nvfp4_byte_count_is_4p5_bits(golden):
    vals = {r[0]: float(r[1]) for r in golden("nvfp4_accounting.txt")}
    for n in (16, 4096, 4096 * 2048):
        nbytes = (n + 1) // 2 + (n + 15) // 16 + 4
        assert (nbytes - 4) * 8 / n == vals["bits_per_value"]
        assert round(16 / ((nbytes - 4) * 8 / n), 2) == vals["gain_vs_fp16"]
    q = O.nvfp4_pack(np.ones(64, np.float32))
    assert q.codes.nbytes + q.scales.nbytes + 4 == 64 // 2 + 64 // 16 + 4


def test_nvfp4_rejects_non_finite():
    for bad in (np.nan, np.inf, -np.inf):
        x = np.ones(20, np.float32)
        x[5] = bad
        with pytest.raises(ValueError):
            O.nvfp4_pack(x)


def test_nvfp4_zero_tensor_and_negative_zero():
    q = O.nvfp4_pack(np.zeros(33, np.float32))
    assert q.ts == 1.0 and np.all(q.scales == 0) and np.all(q.codes == 0)
    x = np.zeros(16, np.float32)
    x[0] = -0.0
    x[1] = 1.0
    q = O.nvfp4_pack(x)
    assert _codes_of(q)[0] == 8  # sign kept on -0
    y = O.nvfp4_unpack(q)
    assert np.signbit(y[0]) and y[0] == 0


def test_half_decode_matches_numpy_all_codes():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.half_value(int(b)) for b in bits])
    r = ref
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])
