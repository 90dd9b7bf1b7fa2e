"""Seeded random group shapes through dict_group_forward against the oracle
(Eq. (1) of "DictLLM: Shared Dictionaries for Post-Training Compression",
Y_l = (X_l D_g) C_l for every layer of a group), as a net under the
hand-picked cases of the other tests: stacked rows from 1 to 280 (decode,
the VALU dot products, the MFMA tiles), ragged d_in, k and d_out, densities
from 2% to 60%, f16 or NVFP4 dictionaries and f16, FP8, INT8 or NVFP4
coefficients.  Every shape is drawn from one fixed seed, so a failure names
a case that can be rerun.  Bound: max|Y_gpu - Y_ref| <= 2e-3 * max|Y_ref|."""
import numpy as np
import pytest

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
