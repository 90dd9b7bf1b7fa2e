"""GPU parity of the factored projection Y_l = (X_l D_g) C_l against the
oracle, through the C ABI, on the seeded workloads (full sizes where the
oracle is quick, sampled tokens otherwise) and on edge cases.

Bound: max|Y_gpu - Y_ref| <= 2e-3 * max|Y_ref| (fp32 accumulation, fp16 or
fp32 storage; for NVFP4 factors the reference uses the oracle's own
dequantised factors)."""
import numpy as np
import pytest
import torch

import oracle as O
from dictionary_factored_sparse_amd import binding as B
from dictionary_factored_sparse_amd import synth
from tests.gpu_helpers import DEV, assert_close, device_group, oracle_group, say

pytestmark = pytest.mark.gpu


def _run_group(g, nvfp4=False, ydtype=torch.float16):
    D, Cs, Xs = device_group(g, nvfp4=nvfp4)
    Ys = B.dict_group_forward(Xs, D, Cs, ydtype=ydtype)
    torch.cuda.synchronize()
    return Ys, (D, Cs, Xs)


@pytest.mark.parametrize("ydtype", [torch.float32, torch.float16])
def test_tiny_group(ydtype):
    say(f"case: tiny group, Y {ydtype}")
    g = synth.make_group("tiny")
    Ys, _ = _run_group(g, ydtype=ydtype)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"tiny layer {l}")


def test_tiny_group_f16_storage():
    say("case: tiny group stored in f16")
    g = synth.make_group("tiny", wdtype=np.float16, xdtype=np.float16)
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"tiny f16 layer {l}")


def test_qproj_decode_group_full():
    say("case: q_proj decode group (2 x 4096->4096, k=2048, density 0.3, T=1)")
    g = synth.make_group("qproj")
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"qproj layer {l}")


def test_qproj_single_projection_matches_group():
    say("case: dict_proj_forward vs dict_group_forward")
    g = synth.make_group("qproj", n_layers=2)
    D, Cs, Xs = device_group(g)
    Ys = B.dict_group_forward(Xs, D, Cs)
    Y1 = B.dict_proj_forward(Xs[1], D, Cs[1])
    torch.cuda.synchronize()
    assert torch.equal(Ys[1], Y1)


def test_qproj_prefill_full_size():
    # every token of both layers against the oracle (about 45 G multiply-adds
    # in float64 on the host's cores)
    say("case: q_proj prefill (2 x T=2048), all tokens")
    g = synth.make_group("qproj_prefill")
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"prefill layer {l}")


def test_wide_tile_prefill_ragged_sampled():
    # 2 x 4100 stacked rows and k = 2000 make 33 x 8 tiles of 256 x 256 (the
    # wide MFMA tile; the last row and atom tiles are partial) and d_in = 2056
    # leaves a short last K tile of 8.
    say("case: wide-tile prefill, 2 x T=4100, d_in=2056, k=2000 (sampled tokens)")
    g = synth.make_group("qproj", d_in=2056, d_out=272, k=2000, T=4100, n_layers=2)
    Ys, _ = _run_group(g)
    rows = np.array([0, 1, 31, 255, 256, 257, 2047, 3839, 3840, 4091, 4092, 4095, 4096, 4099])
    for l, ref in enumerate(oracle_group(g, rows=rows)):
        assert_close(Ys[l][torch.from_numpy(rows).to(DEV)], ref, f"wide layer {l}")


@pytest.mark.parametrize("T", [17, 100, 300])
def test_prefill_ragged_tiles_full(T):
    say(f"case: mid-size prefill T={T} (MFMA + SpMM, ragged tiles)")
    g = synth.make_group("qproj", d_in=512, d_out=400, k=320, T=T, n_layers=2)
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"T={T} layer {l}")


@pytest.mark.parametrize("d_in,k", [(56, 40), (120, 72), (192, 100), (200, 136), (1032, 264)])
def test_mfma_k_tail_and_short_pipelines(d_in, k):
    # d_in % 64 != 0 leaves a short last K tile (zeroed past d_in in LDS);
    # d_in = 192 is three whole tiles (one pass of the pipelined loop);
    # d_in < 64 and < 128 run the K pipeline with one and two tiles; M = 80
    # and N = k leave ragged row and atom tiles.
    say(f"case: MFMA X.D with d_in={d_in}, k={k}, 2 x T=40")
    g = synth.make_group("qproj", d_in=d_in, d_out=96, k=k, T=40, n_layers=2)
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"d_in={d_in} layer {l}")


@pytest.mark.parametrize("ptype", ["gate", "down"])
def test_mlp_group_b1_full(ptype):
    say(f"case: MLP {ptype} group of 4, T=1")
    g = synth.make_group("mlp", ptype=ptype)
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"mlp {ptype} layer {l}")


@pytest.mark.parametrize("ptype", ["up", "down"])
def test_mlp_group_b16_full(ptype):
    say(f"case: MLP {ptype} group of 4, T=16 (64 stacked rows, MFMA)")
    g = synth.make_group("mlp", ptype=ptype, T=16)
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"mlp b16 {ptype} layer {l}")


@pytest.mark.parametrize("ptype", ["q", "gate", "down"])
def test_stack_nvfp4_group_b1(ptype):
    say(f"case: NVFP4 {ptype} group of 2, T=1")
    g = synth.make_group("stack_nvfp4", ptype=ptype, group=3)
    Ys, _ = _run_group(g, nvfp4=True)
    for l, ref in enumerate(oracle_group(g, nvfp4=True)):
        assert_close(Ys[l], ref, f"nvfp4 {ptype} layer {l}")


@pytest.mark.parametrize("T", [3, 40])
def test_nvfp4_small_and_prefill(T):
    say(f"case: NVFP4 factors, T={T}")
    g = synth.make_group("stack_nvfp4", d_in=512, d_out=352, k=256, T=T)
    Ys, _ = _run_group(g, nvfp4=True)
    for l, ref in enumerate(oracle_group(g, nvfp4=True)):
        assert_close(Ys[l], ref, f"nvfp4 T={T} layer {l}")


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 9, 16])
def test_gemv_row_tiles(R):
    say(f"case: VALU path with {R} stacked rows")
    g = synth.make_group("qproj", d_in=1024, d_out=256, k=192, T=R, n_layers=1)
    Ys, _ = _run_group(g)
    assert_close(Ys[0], oracle_group(g)[0], f"rows={R}")


def test_ragged_dims_on_valu_path():
    say("case: d_in=100 (ragged chunk), d_out=37, k=40, ldx padded")
    rng = np.random.default_rng(9)
    d_in, d_out, k, T = 100, 37, 40, 3
    Dn = rng.standard_normal((k, d_in)).astype(np.float16)
    Dpad = np.zeros((k, 104), np.float16)
    Dpad[:, :d_in] = Dn
    Cd = synth.coefficients(rng, k, d_out, 0.4, np.float16)
    X = rng.standard_normal((T, d_in)).astype(np.float16)
    Xpad = np.zeros((T, 104), np.float16)
    Xpad[:, :d_in] = X
    Dt = torch.from_numpy(Dpad).to(DEV)
    D = B.DeviceDict(d_in, k, data=Dt)
    c = B.to_device_csc(Cd, DEV)
    Xt = torch.from_numpy(Xpad).to(DEV)[:, :d_in]
    Y = B.dict_proj_forward(Xt, D, c)
    torch.cuda.synchronize()
    ref = O.forward(X, Dn, d_in, O.pack_csc(Cd))
    assert_close(Y, ref, "ragged")


def test_density_zero_and_empty_columns_exact():
    say("case: density 0 and empty columns give exact zeros")
    g = synth.make_group("qproj", d_in=256, d_out=96, k=64, T=2, n_layers=2, density=0.0)
    Ys, _ = _run_group(g)
    assert all(bool((Y == 0).all()) for Y in Ys)
    g = synth.make_group("qproj", d_in=256, d_out=96, k=64, T=2, n_layers=1, density=0.5)
    g.Cs[0][:, [0, 5, 95]] = 0
    Ys, _ = _run_group(g)
    assert bool((Ys[0][:, [0, 5, 95]] == 0).all())
    assert_close(Ys[0], oracle_group(g)[0], "empty columns")


def test_density_one_and_one_entry_per_column():
    say("case: dense C and one entry per column")
    g = synth.make_group("qproj", d_in=256, d_out=130, k=72, T=5, n_layers=1, density=1.0)
    Ys, _ = _run_group(g)
    assert_close(Ys[0], oracle_group(g)[0], "dense C")
    rng = np.random.default_rng(1)
    Cd = np.zeros((72, 130), np.float16)
    Cd[rng.integers(0, 72, 130), np.arange(130)] = rng.standard_normal(130).astype(np.float16) + 3
    g.Cs[0] = Cd
    Ys, _ = _run_group(g)
    assert_close(Ys[0], oracle_group(g)[0], "one entry per column")


def test_sixteen_layer_group():
    say("case: group of 16 layers, T=1")
    g = synth.make_group("qproj", d_in=512, d_out=256, k=128, T=1, n_layers=16)
    Ys, _ = _run_group(g)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"16-layer group layer {l}")


def _wide_dictionary_group(seed, d_in, d_out, k, T, n, density):
    """A group with more atoms than input features (Gaussian atoms), f16
    factors and activations.  Entries at atom k - 1 and atom 0 in every
    tenth column reach both ends of the staged Z tile."""
    rng = np.random.default_rng(seed)
    Dn = synth.dictionary(rng, d_in, k, "gauss", np.float16)
    Cs = []
    for _ in range(n):
        Cd = synth.coefficients(rng, k, d_out, density, np.float16)
        Cd[k - 1, ::10] = np.float16(0.5)
        Cd[0, 5::10] = np.float16(-0.5)
        Cs.append(Cd)
    Xs = [rng.standard_normal((T, d_in)).astype(np.float16) for _ in range(n)]
    D = B.DeviceDict(d_in, k, data=torch.from_numpy(Dn).to(DEV))
    Ys = B.dict_group_forward([torch.from_numpy(X).to(DEV) for X in Xs], D,
                              [B.to_device_csc(Cd, DEV) for Cd in Cs])
    torch.cuda.synchronize()
    refs = O.group_forward(Xs, Dn, d_in, [O.pack_csc(Cd) for Cd in Cs])
    for l in range(n):
        assert_close(Ys[l], refs[l], f"k={k} T={T} layer {l}")


@pytest.mark.parametrize("d_out,T", [(1, 1), (3, 1), (1, 3), (5, 8), (3, 16), (7, 40)])
def test_few_output_columns(d_out, T):
    """Fewer output columns than workgroups: most workgroups of the SpMV get
    an empty run of column quads (they stage Z and end) and the one quad is
    partial; T = 1 runs the one-launch decode with most workgroups holding
    no column, T = 3, 8 and 16 the SpMV's token tiles, T = 40 the SpMM."""
    say(f"case: d_out={d_out}, d_in=256, k=128, 2 layers, T={T}")
    _wide_dictionary_group(100 + 10 * d_out + T, 256, d_out, 128, T, 2, 0.25)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_largest_forward_k(T):
    """k = 16384, the most atoms a forward call accepts.  T = 1: decode;
    T = 5: VALU dot products and SpMV (10 stacked rows); T = 40: MFMA GEMM
    and SpMM (80 stacked rows, 4-token tiles)."""
    say(f"case: k=16384, d_in=128, d_out=200, 2 layers, T={T}")
    _wide_dictionary_group(16384 + T, 128, 200, 16384, T, 2, 0.01)


@pytest.mark.parametrize("k", [3072, 4607, 4608])
def test_prefill_token_tile_sizes(k):
    """The SpMM's token tile follows k: 16 tokens with one lane per column
    (odd and even columns read the two halves of a Z row in opposite order)
    up to k = 4607, 8 tokens from k = 4608.  T = 40 leaves a ragged tile and
    d_out = 301 an odd last column."""
    say(f"case: prefill SpMM token tiles, k={k}, d_in=256, d_out=301, 2 x T=40")
    _wide_dictionary_group(k, 256, 301, k, 40, 2, 0.05)


def test_zero_tokens_is_a_no_op():
    say("case: T=0")
    g = synth.make_group("tiny", T=1)
    D, Cs, Xs = device_group(g)
    X0 = torch.empty(0, g.d_in, dtype=torch.float32, device=DEV)
    Y0 = torch.empty(0, g.d_out, dtype=torch.float32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.dict_group_forward([X0, X0], D, Cs, Ys=[Y0, Y0], ws=ws)
    torch.cuda.synchronize()


def test_xd_and_zc_entry_points():
    say("case: dict_xd_forward then dict_zc_forward")
    g = synth.make_group("qproj", d_in=1024, d_out=512, k=256, T=4, n_layers=2)
    D, Cs, Xs = device_group(g)
    for zdt in (torch.float32, torch.float16):
        Z = B.dict_xd_forward(Xs, D, zdtype=zdt)
        Ys = B.dict_zc_forward(Z, g.T, Cs)
        torch.cuda.synchronize()
        eye = O.pack_csc(np.eye(g.k, dtype=np.float32))
        for l in range(2):
            zref = O.forward(g.Xs[l], g.D, g.d_in, eye)
            assert_close(Z[l * g.T:(l + 1) * g.T], zref, f"Z layer {l} {zdt}")
        for l, ref in enumerate(oracle_group(g)):
            assert_close(Ys[l], ref, f"zc layer {l} {zdt}")


@pytest.mark.parametrize("k,T,cfmt", [(200, 40, "plain"), (203, 100, "plain"), (200, 40, "fp8"),
                                      (203, 33, "nvfp4")])
def test_zc_fp32_z_many_tokens(k, T, cfmt):
    """Y = Z C from an fp32 Z of more than 16 tokens per layer: the SpMV
    passes over the tokens in fp32 tiles (the SpMM takes f16 Z only);
    k = 203 stages the Z rows element by element."""
    say(f"case: dict_zc_forward, fp32 Z, k={k}, 2 x T={T}, C {cfmt}")
    g = synth.make_group("qproj", d_in=512, d_out=300, k=k, T=T, n_layers=2)
    D, Cs, Xs = device_group(g, cfmt=cfmt)
    Z = B.dict_xd_forward(Xs, D, zdtype=torch.float32)
    Ys = B.dict_zc_forward(Z, T, Cs, ydtype=torch.float32)
    torch.cuda.synchronize()
    for l, ref in enumerate(oracle_group(g, cfmt=cfmt)):
        assert_close(Ys[l], ref, f"fp32 Z, k={k}, T={T}, C {cfmt}, layer {l}")


def test_zc_fp32_z_block_coefficients_many_tokens():
    # the same for block-structured C (8-atom blocks, the last one past k)
    say("case: dict_zc_forward, fp32 Z, block-structured C, k=203, 2 x T=40")
    rng = np.random.default_rng(41)
    d_in, k, d_out, T = 256, 203, 150, 40
    Qm, _ = np.linalg.qr(rng.standard_normal((d_in, k)))
    Dt = np.ascontiguousarray((Qm.T * 64 / np.sqrt(d_in)).astype(np.float16))
    Cs = [synth.block_coefficients(rng, k, d_out, 0.5, np.float16) for _ in range(2)]
    Xs = [rng.standard_normal((T, d_in)).astype(np.float16) for _ in range(2)]
    D = B.to_device_dict(Dt, DEV)
    Z = B.dict_xd_forward([torch.from_numpy(x).to(DEV) for x in Xs], D, zdtype=torch.float32)
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to(DEV)) for c in Cs]
    Ys = B.dict_zc_forward(Z, T, Cg, ydtype=torch.float32)
    torch.cuda.synchronize()
    for l in range(2):
        ref = O.forward_bcsc(Xs[l], Dt, d_in, O.pack_bcsc(Cs[l]))
        assert_close(Ys[l], ref, f"fp32 Z, block C, layer {l}")


@pytest.mark.parametrize("d_in,k,T", [(512, 200, 150), (512, 202, 150), (1032, 264, 40),
                                      (1032, 262, 40)])
def test_mfma_output_tile_forms(d_in, k, T):
    """Z = X D on the MFMA path in f32 and f16.  2 x 150 rows take the
    256 x 128 tile (a ragged last row tile); 2 x 40 rows take 64 x 64 tiles
    with K split in four, whose fp32 partials are summed by a second kernel.
    Tiles whose rows are whole 16-byte pieces (k = 200, 264) leave through
    LDS; k = 202 and 262 keep the element stores."""
    say(f"case: MFMA Z tiles, d_in={d_in}, k={k}, 2 x T={T}, f32 and f16 Z")
    g = synth.make_group("qproj", d_in=d_in, d_out=64, k=k, T=T, n_layers=2)
    D, _, Xs = device_group(g)
    eye = O.pack_csc(np.eye(g.k, dtype=np.float32))
    zrefs = [O.forward(g.Xs[l], g.D, g.d_in, eye) for l in range(2)]
    for zdt in (torch.float32, torch.float16):
        Z = B.dict_xd_forward(Xs, D, zdtype=zdt)
        torch.cuda.synchronize()
        for l in range(2):
            assert_close(Z[l * T:(l + 1) * T], zrefs[l], f"Z layer {l} {zdt}")


@pytest.mark.parametrize("d_in,k,T,n", [(56, 40, 9, 2), (1032, 264, 20, 2), (2048, 2000, 32, 2),
                                        (128, 100, 24, 2), (4104, 3072, 16, 4)])
def test_mfma_few_rows(d_in, k, T, n):
    """Z = X D on the MFMA path for 16 < n T <= 64 stacked rows: 64 x 64
    tiles with K split into slices whose fp32 partials the slice sum adds (8
    for k = 2000, none for d_in = 128, whose two K tiles make one slice).
    Ragged atom tiles (k = 40, 100, 264, 2000), K tails of 8 (d_in = 56,
    1032, 4104), f16 and f32 Z."""
    say(f"case: MFMA Z for few rows, d_in={d_in}, k={k}, {n} x T={T}")
    g = synth.make_group("qproj", d_in=d_in, d_out=64, k=k, T=T, n_layers=n)
    assert g.k == k and g.D.shape == (k, d_in)
    D, _, Xs = device_group(g)
    eye = O.pack_csc(np.eye(g.k, dtype=np.float32))
    zrefs = [O.forward(g.Xs[l], g.D, g.d_in, eye) for l in range(n)]
    for zdt in (torch.float32, torch.float16):
        Z = B.dict_xd_forward(Xs, D, zdtype=zdt)
        torch.cuda.synchronize()
        for l in range(n):
            assert_close(Z[l * T:(l + 1) * T], zrefs[l], f"Z layer {l} {zdt}")


def test_repeat_runs_are_bitwise_identical():
    say("case: determinism")
    for wl, T in (("qproj", 1), ("qproj", 64)):
        g = synth.make_group(wl, d_in=2048, d_out=1024, k=512, T=T, n_layers=2)
        D, Cs, Xs = device_group(g)
        a = B.dict_group_forward(Xs, D, Cs)
        b = B.dict_group_forward(Xs, D, Cs)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_graph_replays_match_eager():
    say("case: HIP graph capture of dict_group_forward, replayed with eager work between")
    g = synth.make_group("qproj", d_in=1024, d_out=768, k=512, T=1, n_layers=2)
    D, Cs, Xs = device_group(g)
    Ys = [torch.empty(1, g.d_out, dtype=torch.float16, device=DEV) for _ in range(2)]
    ws = B.workspace(2, 1, D, Cs[0], DEV)
    B.dict_group_forward(Xs, D, Cs, Ys=Ys, ws=ws)
    torch.cuda.synchronize()
    ref = [y.clone() for y in Ys]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.dict_group_forward(Xs, D, Cs, Ys=Ys, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        B.dict_group_forward(Xs, D, Cs, Ys=Ys, ws=ws)
    for i in range(4):
        for y in Ys:
            y.fill_(float(i + 7))        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for y, r in zip(Ys, ref):
            assert torch.equal(y, r), f"replay {i}"


def _both_paths(g, nvfp4=False, dfmt=None, cfmt=None):
    import os
    D, Cs, Xs = device_group(g, nvfp4=nvfp4, dfmt=dfmt, cfmt=cfmt)
    ws = B.workspace(g.n_layers, g.T, D, Cs[0], DEV)
    out = {}
    for path in ("fused", "two"):
        if path == "two":
            os.environ["DFS_DECODE_PATH"] = "two"
        try:
            out[path] = B.dict_group_forward(Xs, D, Cs, ws=ws)
            torch.cuda.synchronize()
        finally:
            os.environ.pop("DFS_DECODE_PATH", None)
        assert B.workspace_error_word(ws) == 0
    return out


@pytest.mark.parametrize("wl,ptype,nvfp4,n", [("qproj", "q", False, 2), ("qproj", "q", False, 1),
                                              ("mlp", "up", False, 4), ("mlp", "down", False, 3),
                                              ("stack_nvfp4", "q", True, 2),
                                              ("stack_nvfp4", "down", True, 2)])
def test_one_launch_decode_matches_two_launch_and_oracle(wl, ptype, nvfp4, n):
    say(f"case: one-launch decode vs two launches, {wl} {ptype} n={n} nvfp4={nvfp4}")
    g = synth.make_group(wl, ptype=ptype, n_layers=n, T=1)
    out = _both_paths(g, nvfp4=nvfp4)
    refs = oracle_group(g, nvfp4=nvfp4)
    for l, ref in enumerate(refs):
        assert_close(out["fused"][l], ref, f"fused layer {l}")
        assert_close(out["two"][l], ref, f"two-launch layer {l}")


@pytest.mark.parametrize("dfmt,cfmt", [("nvfp4", "plain"), ("plain", "nvfp4")])
def test_mixed_precision_factors(dfmt, cfmt):
    # one factor NVFP4, the other f16: the pages' mixed variants (NVFP4 D with
    # FP16 C); both decode paths and the MFMA prefill path
    say(f"case: mixed factors D {dfmt}, C {cfmt}")
    g = synth.make_group("qproj", d_in=1024, d_out=768, k=512, T=1, n_layers=2)
    out = _both_paths(g, dfmt=dfmt, cfmt=cfmt)
    refs = oracle_group(g, dfmt=dfmt, cfmt=cfmt)
    for l, ref in enumerate(refs):
        assert_close(out["fused"][l], ref, f"fused layer {l}")
        assert_close(out["two"][l], ref, f"two-launch layer {l}")
    gp = synth.make_group("qproj", d_in=1024, d_out=768, k=512, T=40, n_layers=2)
    D, Cs, Xs = device_group(gp, dfmt=dfmt, cfmt=cfmt)
    Ys = B.dict_group_forward(Xs, D, Cs)
    torch.cuda.synchronize()
    for l, ref in enumerate(oracle_group(gp, dfmt=dfmt, cfmt=cfmt)):
        assert_close(Ys[l], ref, f"prefill layer {l}")


@pytest.mark.parametrize("cfmt", ["fp8", "int8"])
@pytest.mark.parametrize("dfmt", ["nvfp4", "plain"])
def test_8bit_coefficients_every_path(dfmt, cfmt):
    # Table 4's mixed-precision pairs (NVFP4 D with FP8 or INT8 C), and f16 D
    # with the same codes: one-launch and two-launch decode, stacked-row SpMV
    # (fp32 and f16 Z tiles), prefill SpMM with ragged token and column tiles
    say(f"case: 8-bit coefficients, D {dfmt}, C {cfmt}")
    g = synth.make_group("qproj", d_in=1024, d_out=776, k=512, T=1, n_layers=2)
    out = _both_paths(g, dfmt=dfmt, cfmt=cfmt)
    refs = oracle_group(g, dfmt=dfmt, cfmt=cfmt)
    for l, ref in enumerate(refs):
        assert_close(out["fused"][l], ref, f"fused layer {l}")
        assert_close(out["two"][l], ref, f"two-launch layer {l}")
    # T = 16 at k = 2048: the SpMV stages Z as f16 (an fp32 tile exceeds 64 KiB)
    for T, k, d_in in ((3, 512, 1024), (16, 2048, 2048), (40, 512, 1024)):
        say(f"  T={T} k={k}")
        gp = synth.make_group("qproj", d_in=d_in, d_out=776, k=k, T=T, n_layers=2)
        assert gp.k == k
        D, Cs, Xs = device_group(gp, dfmt=dfmt, cfmt=cfmt)
        Ys = B.dict_group_forward(Xs, D, Cs)
        torch.cuda.synchronize()
        for l, ref in enumerate(oracle_group(gp, dfmt=dfmt, cfmt=cfmt)):
            assert_close(Ys[l], ref, f"T={T} layer {l}")


@pytest.mark.parametrize("cfmt", ["fp8", "int8"])
def test_8bit_coefficients_full_size_decode(cfmt):
    # the q_proj decode group at full size with an NVFP4 dictionary, and the
    # MLP down group (d_in = 11008: X in three register passes) with f16 D
    say(f"case: q_proj group NVFP4 D + {cfmt} C, full size")
    g = synth.make_group("qproj", T=1, n_layers=2)
    out = _both_paths(g, dfmt="nvfp4", cfmt=cfmt)
    for l, ref in enumerate(oracle_group(g, dfmt="nvfp4", cfmt=cfmt)):
        assert_close(out["fused"][l], ref, f"qproj fused layer {l}")
        assert_close(out["two"][l], ref, f"qproj two-launch layer {l}")
    say(f"case: MLP down group f16 D + {cfmt} C, full size")
    g = synth.make_group("mlp", ptype="down", n_layers=2, T=1)
    out = _both_paths(g, cfmt=cfmt)
    for l, ref in enumerate(oracle_group(g, cfmt=cfmt)):
        assert_close(out["fused"][l], ref, f"down fused layer {l}")


def test_one_launch_decode_x_and_z_lds_regions():
    # The one-launch decode keeps X rows and the received Z side by side in
    # LDS; the MLP down group of 4 fills the most of it (96 KiB of X rows in
    # three passes, 48 KiB of Z).  An earlier layout laid Z over X there, and
    # a missing barrier once let a wave overwrite X under a slower wave of
    # its workgroup (wrong Z for its atoms, only now and then); both shapes
    # are run repeatedly against the oracle.
    for n, cfmt in ((2, "fp8"), (4, "plain")):
        say(f"case: one-launch decode, MLP down n={n}, C {cfmt}, 8 launches")
        g = synth.make_group("mlp", ptype="down", n_layers=n, T=1)
        D, Cs, Xs = device_group(g, cfmt=cfmt)
        refs = oracle_group(g, cfmt=cfmt)
        ws = B.workspace(n, 1, D, Cs[0], DEV)
        for it in range(8):
            Ys = B.dict_group_forward(Xs, D, Cs, ws=ws)
            torch.cuda.synchronize()
            assert B.workspace_error_word(ws) == 0
            for l, ref in enumerate(refs):
                assert_close(Ys[l], ref, f"n={n} launch {it} layer {l}")


def test_one_launch_decode_repeated_launches_identical():
    say("case: one-launch decode, 50 back-to-back launches on one workspace")
    g = synth.make_group("qproj", d_in=2048, d_out=3000, k=1024, T=1, n_layers=2)
    D, Cs, Xs = device_group(g)
    ws = B.workspace(2, 1, D, Cs[0], DEV)
    first = [y.clone() for y in B.dict_group_forward(Xs, D, Cs, ws=ws)]
    Ys = [torch.empty_like(y) for y in first]
    for _ in range(50):
        B.dict_group_forward(Xs, D, Cs, Ys=Ys, ws=ws)
    torch.cuda.synchronize()
    assert B.workspace_error_word(ws) == 0
    for y, f in zip(Ys, first):
        assert torch.equal(y, f)
    for l, ref in enumerate(oracle_group(g)):
        assert_close(first[l], ref, f"layer {l}")
