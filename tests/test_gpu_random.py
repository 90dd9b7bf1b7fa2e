"""Seeded random group shapes through dict_group_forward against the oracle
(Eq. (1) of "DictLLM: Shared Dictionaries for Post-Training Compression",
Y_l = (X_l D_g) C_l for every layer of a group), as a net under the
hand-picked cases of the other tests: stacked rows from 1 to 280 (decode,
the VALU dot products, the MFMA tiles), ragged d_in, k and d_out, densities
from 2% to 60%, f16 or NVFP4 dictionaries and f16, FP8, INT8 or NVFP4
coefficients; the same for several dictionaries over one input
(dict_multi_forward) and for block-structured coefficients.  Every shape is
drawn from one fixed seed, so a failure names a case that can be rerun.  Bound: max|Y_gpu - Y_ref| <= 2e-3 * max|Y_ref|."""
import numpy as np
import pytest
import torch

import oracle as O
from dictionary_factored_sparse_amd import binding as B
from dictionary_factored_sparse_amd import synth
from tests.gpu_helpers import assert_close, device_group, oracle_group, say

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(20):
        d_in = int(rng.integers(2, 100)) * 32        # a multiple of 32: NVFP4 D allowed
        k = int(rng.integers(1, min(d_in, 2048) // 8 + 1)) * 8  # k <= d_in (orthonormal atoms)
        d_out = int(rng.integers(1, 800))
        n = int(rng.integers(1, 5))
        T = int(rng.choice([1, 1, 2, 3, 5, 8, 16, 17, 33, 70]))
        density = float(rng.choice([0.02, 0.1, 0.3, 0.6]))
        dfmt = str(rng.choice(["plain", "nvfp4"]))
        cfmt = str(rng.choice(["plain", "plain", "fp8", "int8", "nvfp4"]))
        out.append((i, d_in, k, d_out, n, T, density, dfmt, cfmt))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_group_shapes(case):
    i, d_in, k, d_out, n, T, density, dfmt, cfmt = case
    say(f"case {i}: d_in={d_in} k={k} d_out={d_out} {n} layers x T={T} density={density} "
        f"D {dfmt} C {cfmt}")
    g = synth.make_group("qproj", group=100 + i, d_in=d_in, d_out=d_out, k=k, T=T, n_layers=n,
                         density=density)
    assert g.k == k and g.D.shape == (k, d_in)
    D, Cs, Xs = device_group(g, dfmt=dfmt, cfmt=cfmt)
    Ys = B.dict_group_forward(Xs, D, Cs)
    refs = oracle_group(g, dfmt=dfmt, cfmt=cfmt)
    for l in range(n):
        assert_close(Ys[l], refs[l], f"case {i} layer {l}")


def _multi_cases():
    rng = np.random.default_rng(20261205)
    out = []
    for i in range(8):
        d_in = int(rng.integers(2, 100)) * 32
        k = int(rng.integers(1, min(d_in, 2048) // 8 + 1)) * 8
        d_out = int(rng.integers(1, 900))
        nd = int(rng.integers(2, 4))
        n = int(rng.integers(1, 3))
        T = int(rng.choice([1, 1, 1, 4, 20]))
        fmt = [("plain", "plain"), ("nvfp4", "nvfp4"), ("nvfp4", "plain")][int(rng.integers(0, 3))]
        out.append((i, d_in, k, d_out, nd, n, T) + fmt)
    return out


@pytest.mark.parametrize("case", _multi_cases(), ids=lambda c: f"multi{c[0]}")
def test_random_multi_dictionary_shapes(case):
    # dict_multi_forward (several dictionaries over the same activations:
    # one launch at T = 1, the groups in turn otherwise) against the oracle
    i, d_in, k, d_out, nd, n, T, dfmt, cfmt = case
    say(f"multi case {i}: {nd} dictionaries, d_in={d_in} k={k} d_out={d_out} {n} layers x T={T} "
        f"D {dfmt} C {cfmt}")
    gs = [synth.make_group("qproj", ptype=p, group=200 + i, d_in=d_in, d_out=d_out, k=k, T=T,
                           n_layers=n) for p in ("q", "k", "v")[:nd]]
    for g in gs[1:]:
        g.Xs = gs[0].Xs
    devs = [device_group(g, dfmt=dfmt, cfmt=cfmt) for g in gs]
    Xs = devs[0][2]
    Ys = B.dict_multi_forward(Xs, [d[0] for d in devs], [c for d in devs for c in d[1]])
    for d, g in enumerate(gs):
        for l, ref in enumerate(oracle_group(g, dfmt=dfmt, cfmt=cfmt)):
            assert_close(Ys[d * n + l], ref, f"multi case {i} dictionary {d} layer {l}")


def _block_cases():
    rng = np.random.default_rng(20261206)
    out = []
    for i in range(8):
        d_in = int(rng.integers(1, 64)) * 32
        k = int(rng.integers(1, min(d_in, 2048) // 8 + 1)) * 8
        if i % 3 == 2:
            k -= int(rng.integers(1, 8))  # a last block that reaches past k
        d_out = int(rng.integers(1, 700))
        n = int(rng.integers(1, 4))
        T = int(rng.choice([1, 1, 3, 8, 17, 40]))
        q = float(rng.choice([0.1, 0.3, 0.533, 0.9]))
        out.append((i, d_in, k, d_out, n, T, q))
    return out


@pytest.mark.parametrize("case", _block_cases(), ids=lambda c: f"block{c[0]}")
def test_random_block_structured_shapes(case):
    # blocks of 8 consecutive atoms per column (the packer, then the one-launch
    # decode, the block SpMV or the block SpMM by row count) against the
    # oracle's block forward
    i, d_in, k, d_out, n, T, q = case
    say(f"block case {i}: d_in={d_in} k={k} d_out={d_out} {n} layers x T={T} blocks kept {q}")
    rng = np.random.default_rng(300 + i)
    Qm, _ = np.linalg.qr(rng.standard_normal((d_in, k)))
    Dt = np.ascontiguousarray((Qm.T * 64 / np.sqrt(d_in)).astype(np.float16))
    Cs = [synth.block_coefficients(rng, k, d_out, q, np.float16) for _ in range(n)]
    Xs = [rng.standard_normal((T, d_in)).astype(np.float16) for _ in range(n)]
    D = B.to_device_dict(Dt, "cuda:0")
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to("cuda:0")) for c in Cs]
    Ys = B.dict_group_forward([torch.from_numpy(x).to("cuda:0") for x in Xs], D, Cg,
                              ydtype=torch.float32)
    for l in range(n):
        ref = O.forward_bcsc(Xs[l], Dt, d_in, O.pack_bcsc(Cs[l]))
        assert_close(Ys[l], ref, f"block case {i} layer {l}")
