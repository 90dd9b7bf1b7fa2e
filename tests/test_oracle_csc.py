"""Pins of the oracle's CSC packer (CPU only).

The packer keeps, per output column, the rows whose entry is nonzero, in
ascending row order ("DictLLM: Shared Dictionaries for Post-Training
Compression", Algorithm 2: export of codes and support, zeros preserved).
Pinned against scipy.sparse's canonical CSC of the same dense matrix (a
library routine), the CSC invariants, and a bitwise round trip.
"""
import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
from dictionary_factored_sparse_amd import synth


def _dense_from_csc(c, dtype):
    out = np.zeros((c.k, c.d_out), dtype)
    for j in range(c.d_out):
        s, e = c.colptr[j], c.colptr[j + 1]
        out[c.rowidx[s:e], j] = c.vals[s:e]
    return out


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
@pytest.mark.parametrize("shape,density", [((128, 256), 0.25), ((300, 77), 0.5), ((1, 5), 1.0),
                                           ((64, 64), 0.0), ((513, 129), 0.03)])
def test_pack_csc_matches_scipy(dtype, shape, density):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    Cd = synth.coefficients(rng, shape[0], shape[1], density, dtype)
    c = O.pack_csc(Cd)
    ref = sp.csc_matrix(Cd.astype(np.float32))   # fp16 -> fp32 is exact
    ref.sort_indices()
    assert np.array_equal(c.colptr, ref.indptr.astype(np.int32))
    assert np.array_equal(c.rowidx.astype(np.int64), ref.indices.astype(np.int64))
    assert np.array_equal(c.vals.view(np.uint8), ref.data.astype(dtype).view(np.uint8))


def test_pack_csc_invariants_and_round_trip():
    rng = np.random.default_rng(5)
    Cd = synth.coefficients(rng, 2048, 300, 0.3, np.float16)
    c = O.pack_csc(Cd)
    assert c.colptr[0] == 0
    assert np.all(np.diff(c.colptr) >= 0)
    assert c.nnz == np.count_nonzero(Cd)
    assert np.all(c.rowidx < 2048)
    for j in range(c.d_out):
        r = c.rowidx[c.colptr[j]:c.colptr[j + 1]].astype(np.int64)
        assert np.all(np.diff(r) > 0)
    back = _dense_from_csc(c, np.float16)
    assert np.array_equal(back.view(np.uint16), Cd.view(np.uint16))
    # per-column nnz of a Bernoulli(0.3) mask over k = 2048 rows is
    # Binomial(2048, 0.3): mean 614.4, sd 20.7
    counts = np.diff(c.colptr)
    assert abs(counts.mean() - 614.4) < 3 * 20.7 / np.sqrt(c.d_out) + 0.5
    assert abs(counts.std() - 20.74) < 3.0


def test_pack_csc_signed_zero_dropped_nan_kept():
    Cd = np.zeros((4, 3), np.float32)
    Cd[0, 0] = -0.0
    Cd[1, 0] = np.nan
    Cd[2, 1] = 2.5
    Cd[3, 2] = -1.0
    c = O.pack_csc(Cd)
    assert list(c.colptr) == [0, 1, 2, 3]
    assert list(c.rowidx) == [1, 2, 3]
    assert np.isnan(c.vals[0]) and c.vals[1] == 2.5 and c.vals[2] == -1.0


def test_pack_csc_max_k_uses_full_uint16_range():
    k = 65536
    Cd = np.zeros((k, 2), np.float16)
    Cd[[0, 1, 65535], 0] = 1.0
    Cd[65534, 1] = -2.0
    c = O.pack_csc(Cd)
    assert list(c.rowidx) == [0, 1, 65535, 65534]
    assert list(c.colptr) == [0, 3, 4]
