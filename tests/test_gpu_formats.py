"""GPU parity of the NVFP4 codec and the CSC packer: bit-exact against the
oracle (integer and byte outputs must be identical)."""
import numpy as np
import pytest
import torch

import oracle as O
from dictionary_factored_sparse_amd import binding as B
from dictionary_factored_sparse_amd import synth
from tests.gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def _gpu_pack(x: np.ndarray):
    q = B.nvfp4_pack(torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV))
    torch.cuda.synchronize()
    n = x.size
    return (q.codes[: (n + 1) // 2].cpu().numpy(), q.scales[: (n + 15) // 16].cpu().numpy(),
            float(q.ts.cpu().item()), q)


def test_unpack_all_code_bytes_and_scales_bit_exact():
    say("case: nvfp4_unpack all 256 code bytes x 127 scales")
    codes = np.tile(np.arange(256, dtype=np.uint8), 127 * 8 // 256 * 2 + 2)[: 127 * 8]
    scales = np.arange(127, dtype=np.uint8)           # every finite non-negative E4M3
    n = 127 * 16
    for ts in (1.0, 0.0123, 3.0e-6, 1.0e-38):
        ts = float(np.float32(ts))
        q = B.DeviceNVFP4(torch.from_numpy(np.concatenate([codes, np.zeros(8, np.uint8)])).to(DEV),
                          torch.from_numpy(scales).to(DEV),
                          torch.tensor([ts], dtype=torch.float32, device=DEV), n)
        got = B.nvfp4_unpack(q).cpu().numpy()
        ref = O.nvfp4_unpack(O.NVFP4(codes, scales, ts, n))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), ts


@pytest.mark.parametrize("n,kind", [(1, "normal"), (15, "normal"), (16, "normal"), (17, "normal"),
                                    (1000, "heavy"), (4096 * 16 + 5, "normal"),
                                    (64, "grid"), (333, "zeros"), (2048, "tiny"), (777, "huge")])
def test_pack_bit_exact(n, kind):
    say(f"case: nvfp4_pack n={n} kind={kind}")
    rng = np.random.default_rng(n + len(kind))
    if kind == "normal":
        x = rng.standard_normal(n).astype(np.float32)
    elif kind == "heavy":
        x = (rng.standard_normal(n) * np.exp(rng.uniform(-12, 12, n))).astype(np.float32)
    elif kind == "grid":
        # exact grid points and midpoints times a power of two: exercises ties
        g = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6],
                     np.float32)
        x = np.concatenate([g, -g, g * 4, -g / 8]).astype(np.float32)
    elif kind == "zeros":
        x = rng.standard_normal(n).astype(np.float32)
        x[::3] = 0.0
        x[1::3] = -0.0
        x[:32] = 0.0
    elif kind == "tiny":
        x = (rng.standard_normal(n) * 1e-37).astype(np.float32)   # subnormal tensor scale
    else:
        x = (rng.standard_normal(n) * 1e37).astype(np.float32)
    codes, scales, ts, _ = _gpu_pack(x)
    ref = O.nvfp4_pack(x)
    assert np.float32(ts).view(np.uint32) == np.float32(ref.ts).view(np.uint32)
    assert np.array_equal(scales, ref.scales)
    assert np.array_equal(codes, ref.codes)


def test_pack_of_qproj_coefficients_bit_exact():
    say("case: nvfp4_pack of a 2048x4096 Bernoulli(0.25) coefficient matrix")
    g = synth.make_group("stack_nvfp4", ptype="q", n_layers=1, T=1)
    x = g.Cs[0][g.Cs[0] != 0].astype(np.float32)
    codes, scales, ts, _ = _gpu_pack(x)
    ref = O.nvfp4_pack(x)
    assert ts == ref.ts
    assert np.array_equal(scales, ref.scales) and np.array_equal(codes, ref.codes)


def _ws_bytes(n):
    import ctypes as C
    b = C.c_size_t(0)
    assert B.lib().nvfp4_pack_workspace_size(n, C.byref(b)) == 0
    return b.value


def test_pack_rejects_non_finite_and_writes_nothing():
    say("case: nvfp4_pack with NaN / Inf")
    for bad in (np.nan, np.inf):
        x = np.ones(100, np.float32)
        x[37] = bad
        q = B.DeviceNVFP4.empty(100, DEV)
        q.codes.fill_(0xAB)
        ws = torch.empty(_ws_bytes(100), dtype=torch.uint8, device=DEV)
        xt = torch.from_numpy(x).to(DEV)
        st = B.lib().nvfp4_pack(xt.data_ptr(), 100, q.nv(), ws.data_ptr(), ws.numel(),
                                torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == 1
        assert bool((q.codes == 0xAB).all())


def test_pack_empty_tensor_sets_unit_scale():
    say("case: nvfp4_pack n=0")
    q = B.DeviceNVFP4.empty(0, DEV)
    ws = torch.empty(_ws_bytes(0), dtype=torch.uint8, device=DEV)
    st = B.lib().nvfp4_pack(None, 0, q.nv(), ws.data_ptr(), ws.numel(),
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and q.ts.item() == 1.0


def _gpu_csc(Cd):
    c = B.dict_pack_csc(torch.from_numpy(Cd).to(DEV))
    torch.cuda.synchronize()
    return (c.colptr.cpu().numpy(), c.rowidx[: c.nnz].cpu().numpy().view(np.uint16),
            c.vals[: c.nnz].cpu().numpy(), c.nnz)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("k,d_out,density", [(128, 256, 0.25), (2048, 4096, 0.3), (3072, 11008, 0.2),
                                             (65, 7, 0.5), (1, 300, 1.0), (300, 1, 0.9),
                                             (64, 64, 0.0)])
def test_pack_csc_bit_exact(dtype, k, d_out, density):
    say(f"case: dict_pack_csc {np.dtype(dtype).name} k={k} d_out={d_out} density={density}")
    rng = np.random.default_rng(k * 31 + d_out)
    Cd = synth.coefficients(rng, k, d_out, density, dtype)
    colptr, rowidx, vals, nnz = _gpu_csc(Cd)
    ref = O.pack_csc(Cd)
    assert nnz == ref.nnz
    assert np.array_equal(colptr, ref.colptr)
    assert np.array_equal(rowidx, ref.rowidx)
    assert np.array_equal(vals.view(np.uint8), ref.vals.view(np.uint8))


def test_pack_csc_special_values_and_max_k():
    say("case: dict_pack_csc with -0, NaN, subnormals, k = 65536")
    k = 65536
    Cd = np.zeros((k, 3), np.float16)
    Cd[[0, 1, 65535], 0] = [1.0, np.nan, -2.0]
    Cd[5, 1] = np.float16(-0.0)
    Cd[6, 1] = np.float16(6e-8)      # f16 subnormal
    Cd[65534, 2] = 3.0
    colptr, rowidx, vals, nnz = _gpu_csc(Cd)
    ref = O.pack_csc(Cd)
    assert nnz == ref.nnz == 5
    assert np.array_equal(colptr, ref.colptr)
    assert np.array_equal(rowidx, ref.rowidx)
    assert np.array_equal(vals.view(np.uint16), ref.vals.view(np.uint16))


def test_pack_csc_capacity_too_small():
    say("case: dict_pack_csc capacity error")
    Cd = torch.ones(16, 8, dtype=torch.float16, device=DEV)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=DEV)
    colptr = torch.empty(9, dtype=torch.int32, device=DEV)
    rowidx = torch.full((64,), 7, dtype=torch.int16, device=DEV)
    vals = torch.zeros(64, dtype=torch.float16, device=DEV)
    import ctypes as C
    nnz = C.c_int64(0)
    st = B.lib().dict_pack_csc(Cd.data_ptr(), B.DFS_F16, 16, 8, 8, colptr.data_ptr(),
                               rowidx.data_ptr(), vals.data_ptr(), 64, C.byref(nnz),
                               ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 3 and nnz.value == 128
    torch.cuda.synchronize()
    assert bool((rowidx == 7).all())


# ------------------------------------------------------------ 8-bit codes

def _gpu_quant8(c, kind):
    q = B.csc_quantize8(c, kind)
    torch.cuda.synchronize()
    return q.codes8[: c.nnz].cpu().numpy(), q.col_scale.cpu().numpy()


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("k,d_out,density,spread", [(128, 256, 0.25, 0.0), (2048, 4096, 0.3, 0.0),
                                                    (65, 7, 0.5, 8.0), (300, 1, 0.9, 0.0),
                                                    (64, 64, 0.0, 0.0), (3000, 37, 0.8, 12.0)])
def test_quantize8_bit_exact(kind, dtype, k, d_out, density, spread):
    say(f"case: dict_csc_quantize8 {kind} {np.dtype(dtype).name} k={k} d_out={d_out} "
        f"density={density} spread={spread}")
    rng = np.random.default_rng(k * 7 + d_out)
    Cd = synth.coefficients(rng, k, d_out, density, np.float32)
    if spread:  # columns spread over many binades (subnormal E4M3 codes appear)
        Cd = Cd * np.exp2(rng.uniform(-spread, spread, d_out)).astype(np.float32)[None, :]
    Cd = Cd.astype(dtype)
    c = B.dict_pack_csc(torch.from_numpy(Cd).to(DEV))
    codes, scale = _gpu_quant8(c, kind)
    ref = O.quantize8_csc(O.pack_csc(Cd), kind).vals
    assert np.array_equal(scale.view(np.uint32), ref.col_scale.view(np.uint32))
    assert np.array_equal(codes, ref.codes)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_quantize8_rejects_non_finite_and_writes_nothing(kind):
    say(f"case: dict_csc_quantize8 {kind} with NaN / Inf")
    import ctypes as C
    for bad in (np.nan, -np.inf):
        Cd = np.ones((16, 4), np.float32)
        Cd[5, 2] = bad
        c = B.dict_pack_csc(torch.from_numpy(Cd).to(DEV))
        codes = torch.full((B.dict_csc_capacity(c.nnz),), 0xAB, dtype=torch.uint8, device=DEV)
        scale = torch.full((4,), 7.0, dtype=torch.float32, device=DEV)
        n = C.c_size_t(0)
        assert B.lib().dict_csc_quantize8_workspace_size(4, C.byref(n)) == 0
        ws = torch.empty(n.value, dtype=torch.uint8, device=DEV)
        d = c.desc()
        st = B.lib().dict_csc_quantize8(C.byref(d), B.CODE8[kind], codes.data_ptr(),
                                        scale.data_ptr(), ws.data_ptr(), n.value,
                                        torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == 1
        assert bool((codes == 0xAB).all()) and bool((scale == 7.0).all())
