"""Pins of the oracle's producer steps (CPU only): the inverse of Eq. (6)-(7),
the compensated deletion of Eq. (7), the fixed-inverse pruning of Algorithm 1
and the refit of Eq. (9), all from "DictLLM: Shared Dictionaries for
Post-Training Compression" (technical review), sections "Method II: prune in
coefficient space" and "Method III: refit the dictionary and quantize the
factors".  What fixes them, other than the oracle itself:
  * the pages' worked examples (tests/golden/refit_example.txt,
    tests/golden/obs_example.txt);
  * library routines on special cases: numpy.linalg.inv for the inverse,
    numpy.linalg.lstsq for the undamped refit, and an equality-constrained
    least-squares solve (numpy.linalg.solve on the reduced system) for the
    compensated deletion;
  * closed forms: the saliency c_i^2/P_ii equals delta^T K delta; with a
    diagonal K a deletion moves no other coordinate and scores K_ii c_i^2;
  * brute force of the pruning order on tiny columns.
"""
import itertools

import numpy as np
import pytest

import oracle as O


def _rows(golden, name):
    return {r[0]: [float(x) for x in r[1:]] for r in golden(name)}


def test_refit_worked_example(golden):
    g = _rows(golden, "refit_example.txt")
    W = np.array([g["W_row0"], g["W_row1"]])
    Cm = np.array([g["C_row0"], g["C_row1"]])
    assert np.allclose(np.diag(Cm @ Cm.T), g["gram_diag"])
    assert np.allclose(W @ Cm.T, [g["WCt_row0"], g["WCt_row1"]])
    Dt = O.refit(W, Cm, 0.0)            # atom-major: row a = column a of D
    assert np.allclose(Dt[0], g["D_col0"], atol=1e-12)
    assert np.allclose(Dt[1], g["D_col1"], atol=1e-12)
    err_id = ((W - Cm) ** 2).sum()      # D = I
    err_fit = ((W - Dt.T @ Cm) ** 2).sum()
    assert err_id == g["sq_err_identity"][0]
    assert abs(err_fit - g["sq_err_refit"][0]) < 1e-12


def test_obs_worked_example(golden):
    g = _rows(golden, "obs_example.txt")
    K = np.array([g["K_row0"], g["K_row1"]])
    c = np.array(g["c"])
    i = int(g["delete"][0])
    P = np.linalg.inv(K)
    moved, s = O.obs_delete(P, c, i)
    assert np.allclose(moved, g["c_after"], atol=1e-12)
    plain = np.zeros(2)
    plain[i] = -c[i]
    assert plain @ K @ plain == g["loss_plain"][0]
    assert round(s, 2) == g["loss_compensated"][0]
    delta = moved - c
    assert abs(delta @ K @ delta - s) < 1e-12


def _spd(rng, n, cond=30.0):
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    ev = np.exp(rng.uniform(0, np.log(cond), n))
    return (Q * ev) @ Q.T


def test_deletion_is_the_constrained_minimum():
    # Eq. (7) against an independent route: minimise d^T K d with d_i = -c_i
    # fixed, solving for the other coordinates with numpy
    rng = np.random.default_rng(1)
    for n in (3, 7, 20):
        K = _spd(rng, n)
        P = np.linalg.inv(K)
        c = rng.standard_normal(n)
        for i in (0, n // 2, n - 1):
            moved, s = O.obs_delete(P, c, i)
            rest = [q for q in range(n) if q != i]
            d_rest = -np.linalg.solve(K[np.ix_(rest, rest)], K[rest, i] * -c[i])
            d = np.zeros(n)
            d[i] = -c[i]
            d[rest] = d_rest
            assert np.allclose(moved - c, d, atol=1e-10)
            assert abs(s - d @ K @ d) < 1e-9 * max(1.0, s)
            assert abs(moved[i]) < 1e-12


def test_diagonal_curvature_moves_nothing_else():
    K = np.diag([2.0, 3.0, 0.5])
    c = np.array([1.0, -2.0, 4.0])
    moved, s = O.obs_delete(np.linalg.inv(K), c, 1)
    assert np.array_equal(moved[[0, 2]], c[[0, 2]]) and moved[1] == 0.0
    assert s == 3.0 * 4.0


def test_gram_inverse_matches_numpy_inv():
    rng = np.random.default_rng(2)
    d_in, k, lam = 40, 16, 0.1
    Dt = rng.standard_normal((k, d_in)).astype(np.float32) / 6
    Xc = rng.standard_normal((200, d_in)).astype(np.float32)
    S = (Xc.T @ Xc / 200).astype(np.float32)
    P = O.gram_inverse(Dt, S, lam)
    D = Dt.astype(np.float64).T
    K = D.T @ S.astype(np.float64) @ D + lam * np.eye(k)
    assert np.allclose(P, np.linalg.inv(K), rtol=1e-9, atol=1e-12)
    assert np.allclose(P @ K, np.eye(k), atol=1e-9)


def test_gram_inverse_rejects_indefinite():
    Dt = np.eye(3, dtype=np.float32)
    S = -np.eye(3, dtype=np.float32)
    with pytest.raises(ValueError):
        O.gram_inverse(Dt, S, 0.0)


def test_refit_undamped_is_least_squares_and_damped_solves_eq9():
    rng = np.random.default_rng(3)
    d_in, k, N = 30, 8, 50
    W = rng.standard_normal((d_in, N)).astype(np.float32)
    Cm = (rng.standard_normal((k, N)) * (rng.random((k, N)) < 0.5)).astype(np.float32)
    Dt = O.refit(W, Cm, 0.0)
    # min ||W - D C||_F over D: D^T = lstsq(C^T, W^T)
    ref = np.linalg.lstsq(Cm.T.astype(np.float64), W.T.astype(np.float64), rcond=None)[0]
    assert np.allclose(Dt, ref, atol=1e-9)
    lam = 0.7
    Dt = O.refit(W, Cm, lam)
    C64, W64 = Cm.astype(np.float64), W.astype(np.float64)
    lhs = Dt.T @ (C64 @ C64.T + lam * np.eye(k))
    assert np.allclose(lhs, W64 @ C64.T, atol=1e-9)
    # an atom with no coefficient anywhere: undamped Gram singular, damped fine
    Cz = Cm.copy()
    Cz[3] = 0
    with pytest.raises(ValueError):
        O.refit(W, Cz, 0.0)
    Dz = O.refit(W, Cz, 0.1)
    assert np.allclose(Dz[3], 0.0)


def _brute_prune_column(c32, P32, n_prune):
    # the same steps, written out with numpy and a plain sort key
    k = len(c32)
    pii = np.diag(P32)
    s = (c32 * c32).astype(np.float32) / pii            # fp32 operations
    order = sorted(range(k), key=lambda i: (float(s[i]), i))[:n_prune]
    c = c32.astype(np.float64)
    P = P32.astype(np.float64)
    for i in order:
        c = c - P[:, i] * (c[i] / P[i, i])
    c[order] = 0.0
    keep = np.ones(k, np.uint8)
    keep[order] = 0
    return c, keep


def test_obs_prune_matches_brute_force_and_keeps_count():
    rng = np.random.default_rng(4)
    k, d_out = 24, 9
    P = np.linalg.inv(_spd(rng, k)).astype(np.float32)
    C = rng.standard_normal((k, d_out)).astype(np.float32)
    C[5, 2] = 0.0                       # a zero coefficient scores 0: pruned first
    for n_prune in (0, 1, 12, 24):
        out, keep = O.obs_prune(C, P, n_prune)
        assert np.all(keep.sum(0) == k - n_prune)
        assert np.all(out[keep == 0] == 0.0)
        for j in range(d_out):
            bc, bk = _brute_prune_column(C[:, j], P, n_prune)
            assert np.array_equal(keep[:, j], bk)
            assert np.allclose(out[:, j], bc, atol=1e-12)
        if n_prune:
            assert keep[5, 2] == 0


def test_obs_prune_order_ties_to_lower_row():
    # equal scores: the lower row goes first
    P = np.eye(4, dtype=np.float32)
    C = np.array([[1.0], [-1.0], [1.0], [2.0]], np.float32)
    _, keep = O.obs_prune(C, P, 2)
    assert keep[:, 0].tolist() == [0, 0, 1, 1]


def test_obs_prune_against_the_joint_solution_eq8():
    # Eq. (8): over all moves that zero the support J, the least quadratic
    # loss is c_J^T (E_J^T P E_J)^-1 c_J.  The sequential prune reaches it for
    # one deletion and cannot go below it for more.
    rng = np.random.default_rng(5)
    k = 16
    K = _spd(rng, k, cond=50.0)
    P32 = np.linalg.inv(K).astype(np.float32)
    P = P32.astype(np.float64)
    c = rng.standard_normal((k, 1)).astype(np.float32)
    for n_prune in (1, 4, 8):
        out, keep = O.obs_prune(c, P32, n_prune)
        J = np.flatnonzero(keep[:, 0] == 0)
        cJ = c[J, 0].astype(np.float64)
        s_joint = cJ @ np.linalg.solve(P[np.ix_(J, J)], cJ)
        Kp = np.linalg.inv(P)
        d = out[:, 0] - c[:, 0].astype(np.float64)
        loss = d @ Kp @ d
        if n_prune == 1:
            assert abs(loss - s_joint) < 1e-9 * max(1.0, s_joint)
        else:
            assert loss >= s_joint - 1e-9 * max(1.0, s_joint)
