"""Pins of the oracle's block-structured support (CPU only): blocks of 8
consecutive atoms per column, the variant the Review asks for in "Let the
accelerator constrain the support" ("DictLLM: Shared Dictionaries for
Post-Training Compression").  What fixes it, other than itself:
  * the round trip: expanding the blocks gives back the dense matrix,
    bitwise, and every block holds a nonzero;
  * the forward equals the oracle's CSC forward on the same matrix (already
    pinned against brute force): the extra entries are exact zeros;
  * brute force of the block count.
"""
import numpy as np
import pytest

import oracle as O
from dictionary_factored_sparse_amd import ledger as L
from dictionary_factored_sparse_amd import synth


def _expand(b):
    Cd = np.zeros((b.k + 8, b.d_out), b.vals.dtype)
    for j in range(b.d_out):
        for q in range(b.colptr[j], b.colptr[j + 1]):
            r = 8 * int(b.bidx[q])
            Cd[r:r + 8, j] = b.vals[8 * q:8 * q + 8]
    return Cd[:b.k]


@pytest.mark.parametrize("k,d_out,dtype", [(64, 10, np.float32), (70, 9, np.float16),
                                           (8, 1, np.float16), (1, 3, np.float32)])
@pytest.mark.parametrize("structured", [False, True])
def test_round_trip_and_block_count(k, d_out, dtype, structured):
    rng = np.random.default_rng(k + d_out)
    if structured:
        Cd = synth.block_coefficients(rng, k, d_out, 0.4, dtype)
    else:
        Cd = synth.coefficients(rng, k, d_out, 0.2, dtype)
    b = O.pack_bcsc(Cd)
    assert np.array_equal(_expand(b).view(np.uint8), Cd.view(np.uint8))
    nb = (k + 7) // 8
    pad = np.zeros((nb * 8, d_out), dtype)
    pad[:k] = Cd
    kept = (pad.reshape(nb, 8, d_out) != 0).any(axis=1)       # nb x d_out
    assert b.nblk == kept.sum()
    assert np.array_equal(np.diff(b.colptr), kept.sum(0))
    for j in range(d_out):
        assert np.array_equal(b.bidx[b.colptr[j]:b.colptr[j + 1]], np.flatnonzero(kept[:, j]))
    for q in range(b.nblk):
        assert np.any(b.vals[8 * q:8 * q + 8] != 0)


@pytest.mark.parametrize("structured", [False, True])
def test_forward_equals_csc_forward(structured):
    rng = np.random.default_rng(5)
    d_in, k, d_out, T = 96, 72, 40, 3
    D = (rng.standard_normal((k, d_in)) / 10).astype(np.float32)
    X = rng.standard_normal((T, d_in)).astype(np.float16)
    if structured:
        Cd = synth.block_coefficients(rng, k, d_out, 0.5, np.float16)
    else:
        Cd = synth.coefficients(rng, k, d_out, 0.3, np.float16)
    Yb = O.forward_bcsc(X, D, d_in, O.pack_bcsc(Cd))
    Yc = O.forward(X, D, d_in, O.pack_csc(Cd))
    assert np.array_equal(Yb, Yc)


def test_block_generator_keeps_whole_blocks():
    rng = np.random.default_rng(6)
    Cd = synth.block_coefficients(rng, 64, 50, 0.3, np.float16)
    blocks = Cd.reshape(8, 8, 50)
    nz = (blocks != 0).sum(axis=1)
    assert set(np.unique(nz)) <= {0, 8}


def test_equal_bytes_block_density():
    # a block of 8 f16 values costs 2 + 16 bytes; an unstructured f16 entry 4
    d_out, k = 4096, 2048
    nnz = int(0.30 * k * d_out)
    q = L.bcsc_density_at_equal_bytes(k, d_out, nnz, "f16")
    nblk = int(round(q * (k // 8) * d_out))
    assert abs(L.bcsc_bytes(d_out, nblk, "f16") - L.csc_bytes(d_out, nnz, "f16")) < 18
    assert abs(q - 0.30 * 4 / 2.25) < 1e-3
