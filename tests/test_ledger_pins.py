"""The byte / multiply-add ledger reproduces the pages' worked numbers
(fixtures under tests/golden cite their passages)."""
import math

from dictionary_factored_sparse_amd import ledger as L


def test_eq3_ranks(golden):
    for rho, n, d_in, d_out, k in golden("eq3_rank.txt"):
        assert L.rank_for_budget(float(rho), int(n), int(d_in), int(d_out)) == int(k)


def test_budget_fractions(golden):
    g = {r[0]: (float(r[1]), int(r[2])) for r in golden("budget_fractions.txt")}
    n, d = 2, 4096
    k = 0.8 * n * d * d / (d + n * d)           # Eq. (3) without the floor
    dict_share = d * k / L.group_values(n, d, d, k, 0.0)
    v, dec = g["dict_share_of_factored"]
    assert round(dict_share, dec) == v
    p = 0.194
    frac = L.group_values(n, d, d, k, p) / L.dense_values(n, d, d)
    v, dec = g["retained_fraction_p0.194"]
    assert round(frac, dec) == v
    assert math.isclose(frac, 0.8 * (1 - 2 * p / 3), rel_tol=1e-12)
    v, dec = g["dictionary_floor"]
    assert round(L.group_values(n, d, d, k, 1.0) / L.dense_values(n, d, d), dec) == v


def test_nvfp4_accounting(golden):
    g = {r[0]: (float(r[1]), int(r[2])) for r in golden("nvfp4_accounting.txt")}
    b = L.nvfp4_bits_per_value()
    assert b == g["bits_per_value"][0]
    assert round(16 / b, 2) == g["gain_vs_fp16"][0]
    assert round(1.43 * round(16 / b, 2), 2) == g["gain_at_1.43x"][0]
    # the page multiplies the rounded 3.56 (2 * 16/4.5 itself is 7.11)
    assert round(2 * round(16 / b, 2), 2) == g["gain_at_2x"][0]
    n = 4096 * 2048
    assert (L.nvfp4_bytes(n) - 4) * 8 / n == b


def test_eq12_thresholds(golden):
    for a, b, h, thr, dec in golden("eq12_thresholds.txt"):
        got = L.sparse_saves_bytes_threshold(float(a), float(b), float(h))
        assert round(got, int(dec)) == float(thr)


def test_eq12_with_this_library_format():
    # 16-bit row indices, NVFP4 values: sparse CSC only saves bytes above
    # 16/20.5 = 78% sparsity, so a 25%-dense C is larger than dense NVFP4.
    thr = L.sparse_saves_bytes_threshold(16, 4.5, 0)
    assert round(thr, 3) == 0.780
    k, d_out = 2048, 4096
    nnz = int(0.25 * k * d_out)
    assert L.csc_bytes(d_out, nnz, "nvfp4") > L.nvfp4_bytes(k * d_out)


def test_mac_fraction(golden):
    for n, d_in, d_out, k, p, frac, dec in golden("mac_fraction.txt"):
        n, d_in, d_out, k = int(n), int(d_in), int(d_out), int(k)
        got = L.macs_factored(n, k, d_in, d_out, float(p)) / L.macs_dense(n, d_in, d_out)
        assert round(got, int(dec)) == float(frac)


def test_illustrative_group(golden):
    g = {r[0]: (float(r[1]), int(r[2])) for r in golden("illustrative_group.txt")}
    n, d, k = 4, 4096, 2048
    dense = L.dense_values(n, d, d)
    grp = L.group_values(n, d, d, k, 0.5)
    M = 1e6
    assert round(dense / M, 1) == g["dense_params_M"][0]
    assert round(d * k / M, 1) == g["dictionary_params_M"][0]
    assert round(0.5 * k * d / M, 1) == g["pruned_C_params_M"][0]
    assert round(grp / M, 1) == g["group_params_M"][0]
    assert round(dense / grp, 1) == g["gain"][0]
    # four private two-factor layers (d x r and r x d each) in the same budget
    r = grp / (n * 2 * d)
    assert int(r) == g["private_rank"][0]


def test_group_bytes_of_the_qproj_decode_group():
    # two layers, D fp16 4096 x 2048 read once, C fp16 at ~30% density
    nnz = int(0.3 * 2048 * 4096)
    b = L.group_bytes(d_in=4096, d_out=4096, k=2048, T=1, nnzs=[nnz, nnz], wdtype="f16",
                      cdtype="f16", xdtype="f16", ydtype="f16")
    assert abs(b / 1e6 - 36.98) < 0.05
