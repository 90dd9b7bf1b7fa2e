"""The C ABI library loads without a GPU, exports every symbol declared in
include/dictfs.h, and rejects bad arguments in host code before any HIP call.

Every call here fails validation (or is a T = 0 no-op), so nothing reaches
the GPU even when this file runs on a GPU machine: the pointers passed are
placeholders that are never dereferenced.
"""
import ctypes as C
import os
import re

import pytest

from dictionary_factored_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dictfs.h")

OK, INVALID, UNSUPPORTED, RANGE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5
P = 0x10000  # 16-byte aligned placeholder address, never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:dfs_status|const char\*|int32_t|int64_t)\s+(\w+)\s*\(", src,
                          re.M))


def test_header_declares_the_boundary_calls():
    fns = header_functions()
    for name in ("dict_pack_csc", "dict_proj_forward", "dict_group_forward", "nvfp4_pack",
                 "nvfp4_unpack"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    L = B.lib()
    fns = header_functions()
    assert fns == set(B.SYMBOLS)
    for name in fns:
        assert hasattr(L, name), name
    assert L.dfs_version() == 301
    assert L.dfs_status_str(0) == b"ok"
    assert L.dfs_status_str(6) == b"HIP runtime error"


def _dict(d_in=256, k=128, dtype=B.DFS_F16, data=P, ldd=None, nv=None):
    return B.Dict(d_in, k, dtype, 0, data, d_in if ldd is None else ldd, nv or B.NV())


def _csc(k=128, d_out=64, nnz=100, dtype=B.DFS_F16, colptr=P, rowidx=P, vals=P, nv=None,
         col_scale=None, capacity=None):
    cap = (nnz + 7) // 8 * 8 if capacity is None else capacity
    return B.Csc(k, d_out, nnz, dtype, 0, colptr, rowidx, vals, nv or B.NV(), col_scale, cap)


def _group(n=1, X=P, xdt=B.DFS_F16, T=1, ldx=256, D=None, Cs=None, Y=P, ydt=B.DFS_F16, ldy=64,
           ws=P, ws_bytes=1 << 30):
    D = D or _dict()
    Cs = Cs or [_csc() for _ in range(n)]
    m = max(n, len(Cs))
    xp = (C.c_void_p * m)(*([X] * m))
    yp = (C.c_void_p * m)(*([Y] * m))
    cs = (B.Csc * len(Cs))(*Cs)
    return B.lib().dict_group_forward(n, xp, xdt, T, ldx, C.byref(D), cs, yp, ydt, ldy, ws,
                                      ws_bytes, None)


def test_group_forward_validation():
    assert _group(T=0) == OK                         # empty batch: nothing to do
    assert _group(D=_dict(d_in=0)) == INVALID
    assert _group(D=_dict(k=20000)) == RANGE        # Z must fit in LDS
    assert _group(D=_dict(k=16385)) == RANGE        # one past the largest forward k
    assert _group(D=_dict(data=None)) == INVALID
    assert _group(D=_dict(data=P + 4)) == ALIGN
    assert _group(D=_dict(ldd=100)) == INVALID      # ldd < d_in
    assert _group(D=_dict(ldd=260)) == ALIGN        # rows not 16-byte aligned
    assert _group(D=_dict(dtype=7)) == UNSUPPORTED
    assert _group(X=P + 2) == ALIGN
    assert _group(X=0) == INVALID
    assert _group(ldx=100) == INVALID
    assert _group(xdt=B.DFS_NVFP4) == UNSUPPORTED
    assert _group(ydt=B.DFS_NVFP4) == UNSUPPORTED
    assert _group(ldy=10) == INVALID
    assert _group(Y=0) == INVALID
    # Y and the column pointers need only their element's alignment
    assert _group(Y=P + 1) == ALIGN
    assert _group(Y=P + 2, ydt=B.DFS_F32) == ALIGN
    assert _group(Y=P + 2, ws_bytes=16) == WORKSPACE              # f16 Y: passes
    assert _group(Cs=[_csc(colptr=P + 2)]) == ALIGN
    assert _group(Cs=[_csc(colptr=P + 4)], ws_bytes=16) == WORKSPACE
    assert _group(Cs=[_csc(k=64)]) == INVALID       # k mismatch with D
    assert _group(Cs=[_csc(nnz=-1)]) == INVALID
    assert _group(Cs=[_csc(nnz=1 << 31)]) == RANGE
    assert _group(Cs=[_csc(rowidx=P + 2)]) == ALIGN
    assert _group(Cs=[_csc(colptr=0)]) == INVALID
    assert _group(Cs=[_csc(dtype=5)]) == UNSUPPORTED
    assert _group(n=2, Cs=[_csc(), _csc(d_out=65)]) == INVALID
    assert _group(n=2, Cs=[_csc(), _csc(dtype=B.DFS_F32)]) == UNSUPPORTED
    assert _group(ws=0) == WORKSPACE
    assert _group(ws_bytes=16) == WORKSPACE
    assert _group(n=17, Cs=[_csc()] * 17) == RANGE
    assert _group(n=0, Cs=[_csc()]) == INVALID
    # NVFP4 dictionary: d_in must be a multiple of 32 and ldd == d_in
    nv = B.NV(P, P, P)
    assert _group(D=_dict(d_in=272, dtype=B.DFS_NVFP4, data=None, nv=nv), ldx=272) == UNSUPPORTED
    assert _group(D=_dict(dtype=B.DFS_NVFP4, data=None, nv=B.NV(P + 1, P, P))) == ALIGN
    assert _group(D=_dict(dtype=B.DFS_NVFP4, data=None, nv=B.NV(P, 0, P))) == INVALID
    # 8-bit coefficient codes need their column scales and aligned codes
    for dt in (B.DFS_FP8, B.DFS_INT8):
        assert _group(Cs=[_csc(dtype=dt)]) == INVALID            # no col_scale
        assert _group(Cs=[_csc(dtype=dt, col_scale=P, vals=P + 8)]) == ALIGN
        assert _group(Cs=[_csc(dtype=dt, col_scale=P, vals=0)]) == INVALID
        assert _group(T=0, Cs=[_csc(dtype=dt, col_scale=P)]) == OK
    # the 8-bit types are coefficient types only
    assert _group(D=_dict(dtype=B.DFS_FP8)) == UNSUPPORTED
    assert _group(xdt=B.DFS_INT8) == UNSUPPORTED


def test_quantize8_validation():
    L = B.lib()
    n = C.c_size_t(0)
    assert L.dict_csc_quantize8_workspace_size(0, C.byref(n)) == INVALID
    assert L.dict_csc_quantize8_workspace_size(64, None) == INVALID
    assert L.dict_csc_quantize8_workspace_size(64, C.byref(n)) == OK and n.value >= 64 * 4

    def call(src=None, dt=B.DFS_FP8, codes=P, scale=P, ws=P, wsb=1 << 20):
        src = _csc() if src is None else src
        return L.dict_csc_quantize8(C.byref(src), dt, codes, scale, ws, wsb, None)

    assert L.dict_csc_quantize8(None, B.DFS_FP8, P, P, P, 1 << 20, None) == INVALID
    assert call(dt=B.DFS_F16) == UNSUPPORTED
    assert call(dt=B.DFS_NVFP4) == UNSUPPORTED
    assert call(src=_csc(dtype=B.DFS_NVFP4, nv=B.NV(P, P, P))) == UNSUPPORTED
    assert call(src=_csc(dtype=B.DFS_FP8, col_scale=P)) == UNSUPPORTED   # already codes
    assert call(scale=0) == INVALID
    assert call(codes=0) == INVALID
    assert call(codes=P + 4) == ALIGN
    assert call(src=_csc(vals=P + 2)) == ALIGN
    assert call(src=_csc(colptr=0)) == INVALID
    assert call(src=_csc(k=0)) == INVALID
    assert call(src=_csc(k=70000)) == RANGE
    assert call(ws=0) == WORKSPACE
    assert call(wsb=16) == WORKSPACE


def test_proj_forward_validation():
    L = B.lib()
    D, c = _dict(), _csc()
    assert L.dict_proj_forward(P, B.DFS_F16, 0, 256, C.byref(D), C.byref(c), P, B.DFS_F16, 64,
                               P, 1 << 20, None) == OK
    assert L.dict_proj_forward(P, B.DFS_F16, -1, 256, C.byref(D), C.byref(c), P, B.DFS_F16, 64,
                               P, 1 << 20, None) == INVALID
    assert L.dict_proj_forward(P, B.DFS_F16, 1, 256, None, C.byref(c), P, B.DFS_F16, 64, P,
                               1 << 20, None) == INVALID


def test_pack_csc_validation():
    L = B.lib()
    nnz = C.c_int64(0)
    args = dict(C=P, dt=B.DFS_F16, k=128, d_out=64, ldc=64, colptr=P, rowidx=P, vals=P, cap=10,
                nnz=C.byref(nnz), ws=P, wsb=1 << 20)

    def call(**kw):
        a = {**args, **kw}
        return L.dict_pack_csc(a["C"], a["dt"], a["k"], a["d_out"], a["ldc"], a["colptr"],
                               a["rowidx"], a["vals"], a["cap"], a["nnz"], a["ws"], a["wsb"],
                               None)
    assert call(C=0) == INVALID
    assert call(colptr=0) == INVALID
    assert call(nnz=None) == INVALID
    assert call(dt=B.DFS_NVFP4) == UNSUPPORTED
    assert call(k=0) == INVALID
    assert call(k=65537) == RANGE
    assert call(ldc=10) == INVALID
    assert call(rowidx=0) == INVALID          # rowidx and vals both or neither
    assert call(cap=-1) == INVALID
    assert call(colptr=P + 2) == ALIGN        # int32 column pointers
    assert call(rowidx=P + 2) == ALIGN        # the forward reads 16-byte chunks
    assert call(vals=P + 8) == ALIGN
    assert call(colptr=P + 4, rowidx=P + 32, vals=P + 48, ws=0) == WORKSPACE  # passes
    assert call(rowidx=0, vals=0, colptr=P + 4, ws=0) == WORKSPACE           # count only
    assert call(ws=0) == WORKSPACE
    assert call(wsb=8) == WORKSPACE
    for ca, cb, cc in ((P + 2, P, P), (P, P + 2, P), (P, P, P + 4)):
        assert L.dict_pack_bcsc(P, B.DFS_F16, 128, 64, 64, ca, cb, cc, 16, C.byref(nnz), P,
                                1 << 20, None) == ALIGN
    n = C.c_size_t(0)
    assert L.dict_pack_csc_workspace_size(65536, 11008, C.byref(n)) == OK and n.value > 0
    assert L.dict_pack_csc_workspace_size(65537, 11008, C.byref(n)) == RANGE


def test_nvfp4_validation():
    L = B.lib()
    assert L.nvfp4_pack(P, -1, B.NV(P, P, P), P, 1 << 20, None) == INVALID
    assert L.nvfp4_pack(0, 10, B.NV(P, P, P), P, 1 << 20, None) == INVALID
    assert L.nvfp4_pack(P, 10, B.NV(P + 4, P, P), P, 1 << 20, None) == ALIGN
    assert L.nvfp4_pack(P, 10, B.NV(P, P, 0), P, 1 << 20, None) == INVALID
    assert L.nvfp4_pack(P, 10, B.NV(P, P, P), P, 4, None) == WORKSPACE
    assert L.nvfp4_unpack(B.NV(P, P, P), -5, P, None) == INVALID
    assert L.nvfp4_unpack(B.NV(P, P, P), 0, P, None) == OK
    assert L.nvfp4_unpack(B.NV(P, 0, P), 7, P, None) == INVALID
    n = C.c_size_t(0)
    assert L.nvfp4_pack_workspace_size(1 << 20, C.byref(n)) == OK and n.value >= 256


def test_workspace_sizes():
    L = B.lib()
    D, c = _dict(d_in=4096, k=2048), _csc(k=2048, d_out=4096)
    n = C.c_size_t(0)
    assert L.dict_workspace_size(2, 1, C.byref(D), C.byref(c), C.byref(n)) == OK
    assert n.value >= 2 * 2048 * 4
    assert L.dict_workspace_size(2, 2048, C.byref(D), C.byref(c), C.byref(n)) == OK
    assert n.value >= 2 * 2048 * 2048 * 2
    assert L.dict_workspace_size(17, 1, C.byref(D), C.byref(c), C.byref(n)) == RANGE
    Dn = _dict(d_in=4096, k=2048, dtype=B.DFS_NVFP4, data=None, nv=B.NV(P, P, P))
    assert L.dict_xd_workspace_size(1, 2048, C.byref(Dn), C.byref(n)) == OK
    assert n.value >= 4096 * 2048 * 2      # f16 expansion for the MFMA path
    assert L.dict_xd_workspace_size(1, 1, C.byref(Dn), C.byref(n)) == OK and n.value == 0


def test_csc_capacity_is_whole_chunks():
    L = B.lib()
    for nnz, cap in ((-1, 8), (0, 8), (1, 8), (7, 8), (8, 8), (9, 16), (2516386, 2516392),
                     ((1 << 31) - 1, 1 << 31)):
        assert L.dict_csc_capacity(nnz) == cap, nnz


def test_producer_validation():
    L = B.lib()
    n = C.c_size_t(0)
    D = _dict()
    assert L.dict_gram_inverse_workspace_size(C.byref(D), C.byref(n)) == OK and n.value > 0
    assert L.dict_gram_inverse_workspace_size(C.byref(_dict(k=9000)), C.byref(n)) == RANGE
    assert L.dict_gram_inverse_workspace_size(
        C.byref(_dict(dtype=B.DFS_NVFP4, data=None, nv=B.NV(P, P, P))), C.byref(n)) == UNSUPPORTED

    def gi(D=None, S=P, lds=256, lam=0.1, Pout=P, ldp=128, ws=P, wsb=1 << 30):
        D = D or _dict()
        return L.dict_gram_inverse(C.byref(D), S, lds, lam, Pout, ldp, ws, wsb, None)
    assert gi(S=0) == INVALID
    assert gi(lds=100) == INVALID
    assert gi(ldp=100) == INVALID
    assert gi(lam=-1.0) == INVALID
    assert gi(lam=float("nan")) == INVALID
    assert gi(ws=0) == WORKSPACE
    assert gi(wsb=16) == WORKSPACE
    assert gi(ws=P + 4) == ALIGN

    def pr(k=128, d_out=64, Cp=P, ldc=64, Pp=P, ldp=128, n_prune=10, Co=P, ldo=64, kp=P, ldk=64):
        return L.dict_obs_prune(k, d_out, Cp, ldc, Pp, ldp, n_prune, Co, ldo, kp, ldk, None)
    assert pr(n_prune=129) == INVALID
    assert pr(n_prune=-1) == INVALID
    assert pr(k=9000, ldp=9000) == RANGE
    assert pr(Cp=0) == INVALID
    assert pr(kp=0) == INVALID
    assert pr(ldc=10) == INVALID
    assert pr(ldp=10) == INVALID

    assert L.dict_refit_workspace_size(0, 8, C.byref(n)) == INVALID
    assert L.dict_refit_workspace_size(16, 9000, C.byref(n)) == RANGE

    def rf(d_in=64, N=100, k=32, W=P, ldw=100, Cm=P, ldc=100, lam=0.0, Dt=P, ldd=64, ws=P,
           wsb=1 << 30):
        return L.dict_refit(d_in, N, k, W, ldw, Cm, ldc, lam, Dt, ldd, ws, wsb, None)
    assert rf(W=0) == INVALID
    assert rf(ldw=50) == INVALID
    assert rf(ldd=10) == INVALID
    assert rf(lam=-0.5) == INVALID
    assert rf(k=9000) == RANGE
    assert rf(wsb=8) == WORKSPACE


def test_block_csc_validation():
    L = B.lib()
    assert _group(Cs=[_csc(dtype=B.DFS_F16)]) != UNSUPPORTED
    blk = B.Csc(128, 64, 100, B.DFS_F16, 8, P, P, P, B.NV(), None, 104)
    assert _group(Cs=[blk], T=0) == OK
    assert _group(Cs=[blk], T=17, ws=P + 8) == ALIGN      # any batch: SpMV or SpMM
    bad = B.Csc(128, 64, 100, B.DFS_F16, 4, P, P, P, B.NV(), None, 104)
    assert _group(Cs=[bad]) == UNSUPPORTED                # blocks of 8 only
    nvb = B.Csc(128, 64, 100, B.DFS_NVFP4, 8, P, P, None, B.NV(P, P, P), None, 104)
    assert _group(Cs=[nvb]) == UNSUPPORTED
    assert _group(n=2, Cs=[_csc(), blk]) == UNSUPPORTED   # one format per group
    nb = C.c_int64(0)
    assert L.dict_pack_bcsc(P, B.DFS_NVFP4, 128, 64, 64, P, None, None, 0, C.byref(nb), P,
                            1 << 20, None) == UNSUPPORTED
    assert L.dict_pack_bcsc(P, B.DFS_F16, 128, 64, 32, P, None, None, 0, C.byref(nb), P,
                            1 << 20, None) == INVALID
    assert L.dict_pack_bcsc(P, B.DFS_F16, 128, 64, 64, P, P, None, 0, C.byref(nb), P,
                            1 << 20, None) == INVALID
    assert L.dict_pack_bcsc(P, B.DFS_F16, 128, 64, 64, P, None, None, 0, C.byref(nb), P,
                            8, None) == WORKSPACE


def test_probe_validation():
    # rejected before any launch (no GPU needed)
    L = B.lib()
    assert L.dfs_probe_mfma(0, 1, P, None) == INVALID
    assert L.dfs_probe_mfma(4, 0, P, None) == INVALID
    assert L.dfs_probe_mfma(4, 1, None, None) == INVALID
    assert L.dfs_probe_mfma((1 << 20) + 1, 1, P, None) == RANGE


def _multi(nd=2, n=1, T=1, Ds=None, Cs=None, ws=P, ws_bytes=1 << 30, X=P, Y=P):
    Ds = Ds or [_dict() for _ in range(nd)]
    Cs = Cs or [_csc() for _ in range(max(nd, len(Ds)) * n)]
    xp = (C.c_void_p * n)(*([X] * n))
    yp = (C.c_void_p * len(Cs))(*([Y] * len(Cs)))
    ds = (B.Dict * len(Ds))(*Ds)
    cs = (B.Csc * len(Cs))(*Cs)
    return B.lib().dict_multi_forward(nd, n, xp, B.DFS_F16, T, 256, ds, cs, yp, B.DFS_F16, 64,
                                      ws, ws_bytes, None)


def test_multi_forward_validation():
    # rejected before any launch (no GPU needed)
    assert _multi(T=0) == OK
    assert _multi(nd=0, Ds=[_dict()]) == INVALID
    assert _multi(nd=9, Ds=[_dict()] * 9) == RANGE
    assert _multi(Ds=[_dict(), _dict(k=64)], Cs=[_csc(), _csc(k=64)]) == INVALID  # k differs
    assert _multi(Ds=[_dict(), _dict(dtype=B.DFS_F32)]) == INVALID               # dtype differs
    assert _multi(Cs=[_csc(), _csc(d_out=65)]) == INVALID                        # d_out differs
    assert _multi(Ds=[_dict(), _dict(data=P + 4)]) == ALIGN                      # per-group checks
    assert _multi(Cs=[_csc(), _csc(k=64)]) == INVALID
    assert _multi(X=0) == INVALID
    assert _multi(ws=0) == WORKSPACE
    assert _multi(ws_bytes=16) == WORKSPACE
    n = C.c_size_t(0)
    d, c = _dict(), _csc()
    assert L_size(3, 2, 1, d, c, n) == OK and n.value >= 4096 + 3 * 2 * 128 * 8
    assert L_size(0, 2, 1, d, c, n) == INVALID
    assert L_size(9, 2, 1, d, c, n) == RANGE


def L_size(nd, n, T, d, c, out):
    return B.lib().dict_multi_workspace_size(nd, n, T, C.byref(d), C.byref(c), C.byref(out))


def test_csc_capacity_is_checked():
    # rowidx / vals hold whole 8-entry chunks: capacity >= nnz rounded up to 8
    assert _group(Cs=[_csc(nnz=100, capacity=100)]) == RANGE
    assert _group(Cs=[_csc(nnz=100, capacity=103)]) == RANGE
    assert _group(Cs=[_csc(nnz=100, capacity=104)], ws=P + 8) == ALIGN  # passes the check
    assert _group(Cs=[_csc(nnz=1, capacity=7)]) == RANGE
    assert _group(Cs=[_csc(nnz=0, capacity=0)], ws=P + 8) == ALIGN     # nothing is read
    # the same check guards the half entry point and the multi-dictionary call
    cs = (B.Csc * 1)(_csc(nnz=100, capacity=96))
    yp = (C.c_void_p * 1)(P)
    assert B.lib().dict_zc_forward(1, P, B.DFS_F32, 1, cs, yp, B.DFS_F16, 64, None) == RANGE


def test_zc_forward_validation():
    # Z is read in 16-byte pieces: a Z that dict_xd_forward would refuse is
    # refused here too, before any launch
    L = B.lib()
    cs = (B.Csc * 1)(_csc())
    yp = (C.c_void_p * 1)(P)
    assert L.dict_zc_forward(1, P + 4, B.DFS_F32, 1, cs, yp, B.DFS_F16, 64, None) == ALIGN
    assert L.dict_zc_forward(1, P + 8, B.DFS_F16, 3, cs, yp, B.DFS_F32, 64, None) == ALIGN
    assert L.dict_zc_forward(1, 0, B.DFS_F32, 1, cs, yp, B.DFS_F16, 64, None) == INVALID
    assert L.dict_zc_forward(1, P + 4, B.DFS_F32, 0, cs, yp, B.DFS_F16, 64, None) == OK  # no rows
    assert L.dict_zc_forward(1, P, B.DFS_NVFP4, 1, cs, yp, B.DFS_F16, 64, None) == UNSUPPORTED
    assert L.dict_zc_forward(1, P, B.DFS_F32, 1, cs, yp, B.DFS_F16, 10, None) == INVALID
    assert L.dict_zc_forward(0, P, B.DFS_F32, 1, cs, yp, B.DFS_F16, 64, None) == INVALID


@pytest.mark.parametrize("xdt,ddt,T,n", [(B.DFS_F32, B.DFS_F32, 32, 2), (B.DFS_F32, B.DFS_F16, 32, 2),
                                         (B.DFS_F16, B.DFS_F16, 32, 2), (B.DFS_F16, B.DFS_F32, 9, 2),
                                         (B.DFS_F16, B.DFS_F16, 1, 4), (B.DFS_F32, B.DFS_F16, 1, 3),
                                         (B.DFS_F16, B.DFS_F16, 2048, 2)])
def test_workspace_query_serves_the_forward(xdt, ddt, T, n):
    # the size the query returns is enough for the forward of any activation
    # dtype (the call then fails on the misaligned workspace, after the size
    # check and before any launch), and one byte less is not
    L = B.lib()
    D = _dict(d_in=256, k=128, dtype=ddt, ldd=256)
    c = _csc(k=128, d_out=64)
    nb = C.c_size_t(0)
    assert L.dict_workspace_size(n, T, C.byref(D), C.byref(c), C.byref(nb)) == OK
    ldx = 256
    assert _group(n=n, xdt=xdt, T=T, ldx=ldx, D=D, Cs=[c] * n, ws=P + 8, ws_bytes=nb.value) == ALIGN
    # the forward's own need for these dtypes is at most the query's
    assert _group(n=n, xdt=xdt, T=T, ldx=ldx, D=D, Cs=[c] * n, ws=P + 8,
                  ws_bytes=nb.value - 1) in (ALIGN, WORKSPACE)
    ms = C.c_size_t(0)
    cs = (B.Csc * (2 * n))(*([c] * (2 * n)))
    Ds = (B.Dict * 2)(D, D)
    assert L.dict_multi_workspace_size(2, n, T, Ds, cs, C.byref(ms)) == OK
    xp = (C.c_void_p * n)(*([P] * n))
    yp = (C.c_void_p * (2 * n))(*([P] * (2 * n)))
    assert L.dict_multi_forward(2, n, xp, xdt, T, ldx, Ds, cs, yp, B.DFS_F16, 64, P + 8,
                                ms.value, None) == ALIGN


def test_noalloc_entry_point_rejects_before_any_launch():
    # dict_group_forward_noalloc: the same argument checks as the group
    # forward, then the workspace the shape needs against the library's
    # 64 MiB array -- both on the host, before anything is enqueued
    L = B.lib()

    def na(n=1, T=1, D=None, Cs=None, X=P, ldx=256, xdt=B.DFS_F16):
        D = D or _dict()
        Cs = Cs or [_csc() for _ in range(n)]
        xp = (C.c_void_p * n)(*([X] * n))
        yp = (C.c_void_p * n)(*([P] * n))
        cs = (B.Csc * n)(*Cs)
        return L.dict_group_forward_noalloc(n, xp, xdt, T, ldx, C.byref(D), cs, yp, B.DFS_F16,
                                            64, None)
    assert na(T=0) == OK
    assert na(X=0) == INVALID
    assert na(D=_dict(k=20000)) == RANGE
    assert na(Cs=[_csc(nnz=100, capacity=96)]) == RANGE
    # 16 layers x 2048 tokens against k = 16384 atoms: a 1 GiB Z tile
    big = _dict(d_in=4096, k=16384, ldd=4096)
    assert na(n=16, T=2048, D=big, Cs=[_csc(k=16384) for _ in range(16)], ldx=4096) == WORKSPACE


def test_read_probe_rejects_before_any_launch():
    # dfs_probe_read checks its arguments on the host; none of these enqueue
    L = B.lib()
    assert L.dfs_probe_read(None, 4096, 4, P, None) == INVALID
    assert L.dfs_probe_read(P, 4096, 4, None, None) == INVALID
    assert L.dfs_probe_read(P, 0, 4, P, None) == INVALID
    assert L.dfs_probe_read(P, 4096, 0, P, None) == INVALID
    assert L.dfs_probe_read(P + 8, 4096, 4, P, None) == ALIGN
    assert L.dfs_probe_read(P, 4100, 4, P, None) == ALIGN
    assert L.dfs_probe_read(P, 4096, (1 << 20) + 1, P, None) == RANGE


def test_binding_rejects_layers_that_do_not_share_one_layout():
    # the C calls take one leading dimension and dtype for every layer's X
    # and Y: the binding refuses lists that disagree before any call
    import types

    import torch
    D = B.DeviceDict(64, 16, data=torch.zeros(16, 64, dtype=torch.float16))
    c = types.SimpleNamespace(d_out=32, k=16)
    X = torch.zeros(2, 64, dtype=torch.float16)
    Y = torch.zeros(2, 32, dtype=torch.float16)
    bad_groups = [
        ([X, torch.zeros(2, 72, dtype=torch.float16)[:, :64]], [Y, Y]),  # row strides differ
        ([X, X.float()], [Y, Y]),                                         # dtypes differ
        ([X, X[:1]], [Y, Y]),                                             # token counts differ
        ([X, X], [Y, torch.zeros(32, 2, dtype=torch.float16).t()]),       # transposed view
        ([X[:, :60], X[:, :60]], [Y, Y]),                                 # not d_in columns
        ([X, X], [Y[:, :30], Y[:, :30]]),                                 # not d_out columns
        ([X, X], [Y[:1], Y[:1]]),                                         # Y rows != T
    ]
    for Xs, Ys in bad_groups:
        with pytest.raises(ValueError):
            B.dict_group_forward(Xs, D, [c, c], Ys=Ys)
    with pytest.raises(ValueError):
        B.dict_zc_forward(torch.zeros(16, 4).t(), 2, [c, c], Ys=[Y, Y])   # Z not contiguous
    with pytest.raises(ValueError):
        B.dict_xd_forward([X, X], D, Z=torch.zeros(4, 8))                 # Z not (n*T, k)


C_USER = r"""
#include <stdio.h>
#include <string.h>
#include "dictfs.h"
int main(void) {
  size_t n = 0;
  dfs_dict d;
  dfs_csc c;
  memset(&d, 0, sizeof d);
  memset(&c, 0, sizeof c);
  if (dfs_version() <= 0) return 1;
  if (dict_csc_capacity(13) != 16 || dict_csc_capacity(0) != 8) return 2;
  if (strcmp(dfs_status_str(DFS_E_ALIGN), "misaligned pointer or leading dimension") != 0) return 3;
  /* validation fails before anything reaches a GPU */
  if (dict_workspace_size(1, 1, &d, &c, &n) != DFS_E_INVALID) return 4;
  if (dict_group_forward(0, NULL, DFS_F16, 1, 8, &d, &c, NULL, DFS_F16, 8, NULL, 0, NULL)
      != DFS_E_INVALID) return 5;
  printf("ok\n");
  return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    # the boundary is a C ABI: a C99 program compiles against the header with
    # every warning as an error, links the library and calls its host checks
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    if os.environ.get("DFS_LIB_PATH"):
        pytest.skip("a host-sanitized build of the library links only with the sanitizer runtime")
    src = tmp_path / "use.c"
    src.write_text(C_USER)
    exe = tmp_path / "use"
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-l:" + os.path.basename(B.LIB_PATH), "-Wl,-rpath," + libdir],
                   check=True, capture_output=True, timeout=120)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
