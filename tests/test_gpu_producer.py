"""GPU parity of the producer steps against the oracle, through the C ABI:
the fixed inverse P = (D^T S D + lambda I)^-1 (Eq. (6)-(7)), fixed-inverse
pruning of the coefficient columns (Algorithm 1) and the dictionary refit
(Eq. (9)), from "DictLLM: Shared Dictionaries for Post-Training Compression",
sections "Method II" and "Method III".

Bars: the pruning mask is bit-exact (both sides order the rows by the same
fp32 scores from the same fp32 inputs); real values within
2e-3 * max|reference| (fp32 GEMMs and Gauss-Jordan elimination against the
oracle's float64 Cholesky solves on inputs of condition number below 100).
"""
import numpy as np
import pytest
import torch

import oracle as O
from dictionary_factored_sparse_amd import binding as B
from tests.gpu_helpers import DEV, assert_close, say

pytestmark = pytest.mark.gpu


def _metric(rng, d_in, T=None):
    T = T or 3 * d_in
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    return (X.T @ X / T).astype(np.float32)


def _atoms(rng, k, d_in, dtype):
    Q, _ = np.linalg.qr(rng.standard_normal((d_in, k)))
    return np.ascontiguousarray((Q.T * (1.0 + rng.random((k, 1)))).astype(dtype))  # k x d_in


@pytest.mark.parametrize("d_in,k,dtype", [(256, 128, np.float32), (200, 72, np.float16),
                                          (1024, 512, np.float32)])
def test_gram_inverse(d_in, k, dtype):
    say(f"case: dict_gram_inverse d_in={d_in} k={k} {np.dtype(dtype).name}")
    rng = np.random.default_rng(d_in + k)
    Dt = _atoms(rng, k, d_in, dtype)
    S = _metric(rng, d_in)
    lam = 0.05
    D = B.to_device_dict(Dt, DEV)
    P, err = B.dict_gram_inverse(D, torch.from_numpy(S).to(DEV), lam)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = O.gram_inverse(Dt.astype(np.float32), S, lam)
    assert_close(P, ref, f"P d_in={d_in} k={k}")


def test_gram_inverse_flags_indefinite():
    say("case: dict_gram_inverse on a negative definite matrix")
    Dt = np.eye(8, 16, dtype=np.float32)
    S = -np.eye(16, dtype=np.float32)
    P, err = B.dict_gram_inverse(B.to_device_dict(Dt, DEV), torch.from_numpy(S).to(DEV), 0.0)
    torch.cuda.synchronize()
    assert int(err.item()) != 0


def _spd_inverse(rng, k, cond=30.0):
    Q, _ = np.linalg.qr(rng.standard_normal((k, k)))
    ev = np.exp(rng.uniform(0, np.log(cond), k))
    return ((Q / ev) @ Q.T).astype(np.float32)          # the inverse of an SPD matrix


@pytest.mark.parametrize("k,d_out,n_prune", [(128, 100, 64), (128, 33, 0), (128, 33, 1),
                                             (128, 33, 128), (300, 70, 150), (4, 5, 2)])
def test_obs_prune(k, d_out, n_prune):
    say(f"case: dict_obs_prune k={k} d_out={d_out} n_prune={n_prune}")
    rng = np.random.default_rng(k * 3 + d_out)
    P = _spd_inverse(rng, k)
    C = rng.standard_normal((k, d_out)).astype(np.float32)
    C[rng.random((k, d_out)) < 0.05] = 0.0               # zeros score 0: pruned first
    out, keep = B.dict_obs_prune(torch.from_numpy(C).to(DEV), torch.from_numpy(P).to(DEV),
                                 n_prune)
    torch.cuda.synchronize()
    ref, ref_keep = O.obs_prune(C, P, n_prune)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)
    assert_close(out, ref, f"pruned C k={k}")
    assert bool((out[keep == 0] == 0).all())


def test_obs_prune_full_size_sampled_columns():
    # the q_proj group shape: k = 2048 atoms, 4096 columns, half of each
    # column pruned (the 50% coefficient sparsity of Table 4's model)
    say("case: dict_obs_prune k=2048 d_out=4096 n_prune=1024, sampled columns")
    rng = np.random.default_rng(77)
    k, d_out = 2048, 4096
    A = rng.standard_normal((k, 256)) / 16
    P = (A @ A.T + 0.5 * np.eye(k)).astype(np.float32)   # SPD, positive diagonal
    C = (rng.standard_normal((k, d_out)) / np.sqrt(k)).astype(np.float32)
    out, keep = B.dict_obs_prune(torch.from_numpy(C).to(DEV), torch.from_numpy(P).to(DEV), 1024)
    torch.cuda.synchronize()
    cols = np.array([0, 1, 17, 1000, 2047, 2048, 4000, 4095])
    ref, ref_keep = O.obs_prune(np.ascontiguousarray(C[:, cols]), P, 1024)
    assert np.array_equal(keep.cpu().numpy()[:, cols], ref_keep)
    assert_close(out[:, torch.from_numpy(cols).to(DEV)], ref, "pruned C sampled")
    assert bool((keep.sum(0) == k - 1024).all())


@pytest.mark.parametrize("d_in,N,k,lam", [(256, 384, 128, 0.0), (256, 384, 128, 0.5),
                                          (200, 250, 72, 0.01)])
def test_refit(d_in, N, k, lam):
    say(f"case: dict_refit d_in={d_in} N={N} k={k} lambda={lam}")
    rng = np.random.default_rng(d_in + N + k)
    W = rng.standard_normal((d_in, N)).astype(np.float32)
    Cm = (rng.standard_normal((k, N)) * (rng.random((k, N)) < 0.5)).astype(np.float32)
    Dt, err = B.dict_refit(torch.from_numpy(W).to(DEV), torch.from_numpy(Cm).to(DEV), lam)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = O.refit(W, Cm, lam)
    assert_close(Dt, ref, f"refit d_in={d_in} k={k}")


def test_prune_then_refit_lowers_the_weighted_error():
    # the two steps in sequence on a small group (two layers side by side):
    # the metric-weighted reconstruction error after pruning falls after the
    # refit (Eq. (9) solves that least-squares problem for the kept support)
    say("case: gram inverse -> prune -> refit on a 2-layer group")
    rng = np.random.default_rng(9)
    d_in, d_out, k = 256, 192, 96
    Dt0 = _atoms(rng, k, d_in, np.float32)
    Cs = [(rng.standard_normal((k, d_out)) / np.sqrt(k)).astype(np.float32) for _ in range(2)]
    Ws = [(Dt0.T @ c + 0.01 * rng.standard_normal((d_in, d_out))).astype(np.float32) for c in Cs]
    S = _metric(rng, d_in)
    D = B.to_device_dict(Dt0, DEV)
    P, err = B.dict_gram_inverse(D, torch.from_numpy(S).to(DEV), 1e-3)
    pruned = [B.dict_obs_prune(torch.from_numpy(c).to(DEV), P, k // 2)[0] for c in Cs]
    Cm = torch.cat(pruned, dim=1).contiguous()
    W = torch.from_numpy(np.concatenate(Ws, axis=1)).to(DEV)
    Dt1, err2 = B.dict_refit(W, Cm, 1e-3)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and int(err2.item()) == 0
    Sd = torch.from_numpy(S.astype(np.float64))
    def werr(Dt):
        R = W.double().cpu() - Dt.double().cpu().T @ Cm.double().cpu()
        return float(torch.trace(R.T @ Sd @ R))
    e0 = werr(torch.from_numpy(Dt0))
    e1 = werr(Dt1)
    assert e1 < e0
