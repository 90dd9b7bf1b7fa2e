"""Thin ctypes binding of ``libdictfs.so`` (C ABI in include/dictfs.h).

Argument marshalling only: every step of the projection runs in the HIP
library.  Device memory and streams come from PyTorch (tensors on a ROCm
device; the current torch stream is passed as the hipStream_t).  There is no
fallback: if the library is missing or a call fails, an exception is raised.

The functions carry the C names.  Small holder classes (``DeviceDict``,
``DeviceCSC``, ``DeviceNVFP4``) keep the tensors a descriptor points at alive.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DFS_LIB_PATH selects another build of the same library (the host-sanitized
# build used by the CPU sanitizer test); there is no fallback when it is missing
LIB_PATH = os.environ.get("DFS_LIB_PATH") or os.path.join(_PKG, "libdictfs.so")

DFS_F32, DFS_F16, DFS_NVFP4, DFS_FP8, DFS_INT8 = 0, 1, 2, 3, 4
CODE8 = {"fp8": DFS_FP8, "int8": DFS_INT8}
STATUS = {0: "DFS_OK", 1: "DFS_E_INVALID", 2: "DFS_E_UNSUPPORTED", 3: "DFS_E_RANGE",
          4: "DFS_E_ALIGN", 5: "DFS_E_WORKSPACE", 6: "DFS_E_HIP"}

# symbols declared in include/dictfs.h
SYMBOLS = ("dict_pack_csc_workspace_size", "dict_pack_csc", "nvfp4_pack_workspace_size",
           "nvfp4_pack", "nvfp4_unpack", "dict_workspace_size", "dict_proj_forward",
           "dict_group_forward", "dict_xd_forward", "dict_xd_workspace_size", "dict_zc_forward",
           "dfs_status_str", "dfs_last_hip_error", "dfs_version", "dict_csc_capacity",
           "dict_csc_quantize8_workspace_size", "dict_csc_quantize8",
           "dict_gram_inverse_workspace_size", "dict_gram_inverse", "dict_obs_prune",
           "dict_refit_workspace_size", "dict_refit", "dict_pack_bcsc", "dfs_probe_mfma",
           "dfs_probe_read",
           "dict_multi_workspace_size", "dict_multi_forward", "dict_group_forward_noalloc")


class NV(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("tensor_scale", C.c_void_p)]


class Dict(C.Structure):
    _fields_ = [("d_in", C.c_int32), ("k", C.c_int32), ("dtype", C.c_int32), ("_pad", C.c_int32),
                ("data", C.c_void_p), ("ldd", C.c_int64), ("nv", NV)]


class Csc(C.Structure):
    _fields_ = [("k", C.c_int32), ("d_out", C.c_int32), ("nnz", C.c_int64), ("dtype", C.c_int32),
                ("block_rows", C.c_int32), ("colptr", C.c_void_p), ("rowidx", C.c_void_p),
                ("vals", C.c_void_p), ("nv", NV), ("col_scale", C.c_void_p),
                ("capacity", C.c_int64)]


class DfsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.hip_error = int(lib().dfs_last_hip_error()) if status == 6 else 0
        msg = lib().dfs_status_str(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})"
                         + (f", hipError {self.hip_error}" if self.hip_error else ""))


_lib = None


def lib():
    """Load libdictfs.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        psz = C.POINTER(C.c_size_t)
        sig = {
            "dict_pack_csc_workspace_size": [i32, i32, psz],
            "dict_pack_csc": [vp, i32, i32, i32, i64, vp, vp, vp, i64, C.POINTER(C.c_int64), vp,
                              sz, vp],
            "nvfp4_pack_workspace_size": [i64, psz],
            "nvfp4_pack": [vp, i64, NV, vp, sz, vp],
            "nvfp4_unpack": [NV, i64, vp, vp],
            "dict_workspace_size": [i32, i32, C.POINTER(Dict), C.POINTER(Csc), psz],
            "dict_proj_forward": [vp, i32, i32, i64, C.POINTER(Dict), C.POINTER(Csc), vp, i32,
                                  i64, vp, sz, vp],
            "dict_group_forward": [i32, C.POINTER(vp), i32, i32, i64, C.POINTER(Dict),
                                   C.POINTER(Csc), C.POINTER(vp), i32, i64, vp, sz, vp],
            "dict_xd_forward": [i32, C.POINTER(vp), i32, i32, i64, C.POINTER(Dict), vp, i32, vp,
                                sz, vp],
            "dict_xd_workspace_size": [i32, i32, C.POINTER(Dict), psz],
            "dict_zc_forward": [i32, vp, i32, i32, C.POINTER(Csc), C.POINTER(vp), i32, i64, vp],
            "dict_csc_quantize8_workspace_size": [i32, psz],
            "dict_csc_quantize8": [C.POINTER(Csc), i32, vp, vp, vp, sz, vp],
            "dict_pack_bcsc": [vp, i32, i32, i32, i64, vp, vp, vp, i64, C.POINTER(C.c_int64), vp,
                               sz, vp],
            "dict_gram_inverse_workspace_size": [C.POINTER(Dict), psz],
            "dict_gram_inverse": [C.POINTER(Dict), vp, i64, C.c_float, vp, i64, vp, sz, vp],
            "dict_obs_prune": [i32, i32, vp, i64, vp, i64, i32, vp, i64, vp, i64, vp],
            "dict_refit_workspace_size": [i32, i32, psz],
            "dict_refit": [i32, i32, i32, vp, i64, vp, i64, C.c_float, vp, i64, vp, sz, vp],
            "dfs_probe_mfma": [i32, i32, vp, vp],
            "dfs_probe_read": [vp, i64, i32, vp, vp],
            "dict_multi_workspace_size": [i32, i32, i32, C.POINTER(Dict), C.POINTER(Csc), psz],
            "dict_multi_forward": [i32, i32, C.POINTER(vp), i32, i32, i64, C.POINTER(Dict),
                                   C.POINTER(Csc), C.POINTER(vp), i32, i64, vp, sz, vp],
            "dict_group_forward_noalloc": [i32, C.POINTER(vp), i32, i32, i64, C.POINTER(Dict),
                                           C.POINTER(Csc), C.POINTER(vp), i32, i64, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        L.dfs_status_str.argtypes = [C.c_int]
        L.dfs_status_str.restype = C.c_char_p
        L.dfs_last_hip_error.restype = C.c_int32
        L.dfs_version.restype = C.c_int32
        L.dict_csc_capacity.argtypes = [C.c_int64]
        L.dict_csc_capacity.restype = C.c_int64
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise DfsError(fn, status)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return DFS_F16
    if t.dtype == torch.float32:
        return DFS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows(ts, what: str, width: int | None = None) -> None:
    """The C calls take one pointer per layer and ONE leading dimension and
    dtype for all of them: every tensor must be a 2-D row-major view with
    unit column stride, and all must agree in shape, stride, dtype and
    device."""
    t0 = ts[0]
    for t in ts:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"{what}: 2-D row-major tensors with unit column stride required")
        if (t.shape != t0.shape or t.stride(0) != t0.stride(0) or t.dtype != t0.dtype
                or t.device != t0.device):
            raise ValueError(f"{what}: every layer needs the same shape, row stride, dtype and "
                             "device")
    if width is not None and t0.shape[1] != width:
        raise ValueError(f"{what}: {t0.shape[1]} columns, expected {width}")


def _torch_dt(code: int):
    return {DFS_F16: torch.float16, DFS_F32: torch.float32}[code]


# ----------------------------------------------------------------- holders

@dataclass
class DeviceNVFP4:
    codes: torch.Tensor    # uint8[(n+1)//2]
    scales: torch.Tensor   # uint8[(n+15)//16]
    ts: torch.Tensor       # float32[1]
    n: int

    def nv(self) -> NV:
        return NV(self.codes.data_ptr(), self.scales.data_ptr(), self.ts.data_ptr())

    @staticmethod
    def empty(n: int, device) -> "DeviceNVFP4":
        # codes padded to 16 bytes so 16-byte chunk reads stay in bounds
        nc = ((n + 1) // 2 + 15) // 16 * 16
        return DeviceNVFP4(torch.zeros(max(nc, 16), dtype=torch.uint8, device=device),
                           torch.zeros(max((n + 15) // 16, 1), dtype=torch.uint8, device=device),
                           torch.zeros(1, dtype=torch.float32, device=device), n)


@dataclass
class DeviceDict:
    """D_g stored atom-major: ``data`` is (k, d_in), or ``nv`` holds k*d_in
    NVFP4 elements in that order."""
    d_in: int
    k: int
    data: torch.Tensor | None = None
    nv: DeviceNVFP4 | None = None

    def desc(self) -> Dict:
        if self.nv is not None:
            return Dict(self.d_in, self.k, DFS_NVFP4, 0, None, self.d_in, self.nv.nv())
        return Dict(self.d_in, self.k, _dt(self.data), 0, self.data.data_ptr(),
                    self.data.stride(0), NV())

    @staticmethod
    def from_atoms(atoms: torch.Tensor) -> "DeviceDict":
        assert atoms.dim() == 2 and atoms.stride(1) == 1
        return DeviceDict(atoms.shape[1], atoms.shape[0], data=atoms)


@dataclass
class DeviceCSC:
    k: int
    d_out: int
    nnz: int
    colptr: torch.Tensor          # int32[d_out+1]
    rowidx: torch.Tensor          # uint16 storage (int16 tensor) [>= nnz]
    vals: torch.Tensor | None = None
    nv: DeviceNVFP4 | None = None
    codes8: torch.Tensor | None = None     # uint8[capacity] FP8 / INT8 codes
    col_scale: torch.Tensor | None = None  # float32[d_out]
    code_kind: str | None = None           # "fp8" or "int8"
    block_rows: int = 0                    # 8: colptr/nnz count blocks of 8 atoms

    @property
    def capacity(self) -> int:
        """Entries (blocks, for block_rows = 8) that rowidx and the values
        are allocated for: the smallest of the arrays' lengths."""
        cap = self.rowidx.numel()
        if self.nv is not None:
            cap = min(cap, 2 * self.nv.codes.numel(), 16 * self.nv.scales.numel())
        elif self.codes8 is not None:
            cap = min(cap, self.codes8.numel())
        else:
            cap = min(cap, self.vals.numel() // (self.block_rows or 1))
        return cap

    def desc(self) -> Csc:
        if self.nv is not None:
            return Csc(self.k, self.d_out, self.nnz, DFS_NVFP4, 0, self.colptr.data_ptr(),
                       self.rowidx.data_ptr(), None, self.nv.nv(), None, self.capacity)
        if self.codes8 is not None:
            return Csc(self.k, self.d_out, self.nnz, CODE8[self.code_kind], 0,
                       self.colptr.data_ptr(), self.rowidx.data_ptr(), self.codes8.data_ptr(),
                       NV(), self.col_scale.data_ptr(), self.capacity)
        return Csc(self.k, self.d_out, self.nnz, _dt(self.vals), self.block_rows,
                   self.colptr.data_ptr(), self.rowidx.data_ptr(), self.vals.data_ptr(), NV(),
                   None, self.capacity)

    @property
    def fmt(self) -> str:
        if self.nv is not None:
            return "nvfp4"
        if self.codes8 is not None:
            return self.code_kind
        return "f16" if self.vals.dtype == torch.float16 else "f32"


def dict_csc_capacity(nnz: int) -> int:
    """Entries rowidx/vals must be allocated for (whole 8-entry chunks)."""
    return int(lib().dict_csc_capacity(int(nnz)))


# ----------------------------------------------------------------- packing

def dict_pack_csc(Cd: torch.Tensor, stream=None) -> DeviceCSC:
    """Dense (k, d_out) f16/f32 device tensor -> DeviceCSC (two calls: count,
    then fill into buffers sized from the count)."""
    assert Cd.dim() == 2 and Cd.stride(1) == 1
    k, d_out = Cd.shape
    dev = Cd.device
    ws_n = C.c_size_t(0)
    _check("dict_pack_csc_workspace_size",
           lib().dict_pack_csc_workspace_size(k, d_out, C.byref(ws_n)))
    ws = torch.empty(ws_n.value, dtype=torch.uint8, device=dev)
    colptr = torch.empty(d_out + 1, dtype=torch.int32, device=dev)
    nnz = C.c_int64(0)
    st = _stream(stream)
    _check("dict_pack_csc", lib().dict_pack_csc(Cd.data_ptr(), _dt(Cd), k, d_out, Cd.stride(0),
                                                colptr.data_ptr(), None, None, 0, C.byref(nnz),
                                                ws.data_ptr(), ws_n.value, st))
    n = nnz.value
    cap = dict_csc_capacity(n)
    rowidx = torch.zeros(cap, dtype=torch.int16, device=dev)
    vals = torch.zeros(cap, dtype=Cd.dtype, device=dev)
    _check("dict_pack_csc", lib().dict_pack_csc(Cd.data_ptr(), _dt(Cd), k, d_out, Cd.stride(0),
                                                colptr.data_ptr(), rowidx.data_ptr(),
                                                vals.data_ptr(), rowidx.numel(), C.byref(nnz),
                                                ws.data_ptr(), ws_n.value, st))
    return DeviceCSC(k, d_out, n, colptr, rowidx, vals=vals)


def dict_pack_bcsc(Cd: torch.Tensor, stream=None) -> DeviceCSC:
    """Dense (k, d_out) f16/f32 device tensor -> block-structured DeviceCSC
    (blocks of 8 consecutive atoms per column; count call, then fill)."""
    assert Cd.dim() == 2 and Cd.stride(1) == 1
    k, d_out = Cd.shape
    dev = Cd.device
    ws_n = C.c_size_t(0)
    _check("dict_pack_csc_workspace_size",
           lib().dict_pack_csc_workspace_size(k, d_out, C.byref(ws_n)))
    ws = torch.empty(ws_n.value, dtype=torch.uint8, device=dev)
    colptr = torch.empty(d_out + 1, dtype=torch.int32, device=dev)
    nb = C.c_int64(0)
    st = _stream(stream)
    _check("dict_pack_bcsc", lib().dict_pack_bcsc(Cd.data_ptr(), _dt(Cd), k, d_out, Cd.stride(0),
                                                  colptr.data_ptr(), None, None, 0, C.byref(nb),
                                                  ws.data_ptr(), ws_n.value, st))
    n = nb.value
    cap = dict_csc_capacity(n)
    bidx = torch.zeros(cap, dtype=torch.int16, device=dev)
    vals = torch.zeros(8 * cap, dtype=Cd.dtype, device=dev)
    _check("dict_pack_bcsc", lib().dict_pack_bcsc(Cd.data_ptr(), _dt(Cd), k, d_out, Cd.stride(0),
                                                  colptr.data_ptr(), bidx.data_ptr(),
                                                  vals.data_ptr(), cap, C.byref(nb),
                                                  ws.data_ptr(), ws_n.value, st))
    return DeviceCSC(k, d_out, n, colptr, bidx, vals=vals, block_rows=8)


def nvfp4_pack(x: torch.Tensor, stream=None) -> DeviceNVFP4:
    """fp32 device tensor (any shape, contiguous) -> DeviceNVFP4 of x.numel()."""
    assert x.dtype == torch.float32 and x.is_contiguous()
    n = x.numel()
    q = DeviceNVFP4.empty(n, x.device)
    ws_n = C.c_size_t(0)
    _check("nvfp4_pack_workspace_size", lib().nvfp4_pack_workspace_size(n, C.byref(ws_n)))
    ws = torch.empty(ws_n.value, dtype=torch.uint8, device=x.device)
    _check("nvfp4_pack", lib().nvfp4_pack(x.data_ptr(), n, q.nv(), ws.data_ptr(), ws_n.value,
                                          _stream(stream)))
    return q


def nvfp4_unpack(q: DeviceNVFP4, stream=None) -> torch.Tensor:
    y = torch.empty(q.n, dtype=torch.float32, device=q.codes.device)
    _check("nvfp4_unpack", lib().nvfp4_unpack(q.nv(), q.n, y.data_ptr(), _stream(stream)))
    return y


def csc_to_nvfp4(c: DeviceCSC, stream=None) -> DeviceCSC:
    """Quantise a DeviceCSC's values (CSC order) to NVFP4, support unchanged."""
    v = c.vals[:c.nnz].float().contiguous()
    return DeviceCSC(c.k, c.d_out, c.nnz, c.colptr, c.rowidx, nv=nvfp4_pack(v, stream))


def csc_quantize8(c: DeviceCSC, kind: str, stream=None) -> DeviceCSC:
    """Quantise a DeviceCSC's f16/f32 values to 8-bit codes (``kind`` "fp8"
    or "int8", one scale per column); support shared with ``c``."""
    if kind not in CODE8:
        raise ValueError(kind)
    dev = c.colptr.device
    codes = torch.zeros(dict_csc_capacity(c.nnz), dtype=torch.uint8, device=dev)
    scale = torch.empty(c.d_out, dtype=torch.float32, device=dev)
    ws_n = C.c_size_t(0)
    _check("dict_csc_quantize8_workspace_size",
           lib().dict_csc_quantize8_workspace_size(c.d_out, C.byref(ws_n)))
    ws = torch.empty(ws_n.value, dtype=torch.uint8, device=dev)
    d = c.desc()
    _check("dict_csc_quantize8",
           lib().dict_csc_quantize8(C.byref(d), CODE8[kind], codes.data_ptr(), scale.data_ptr(),
                                    ws.data_ptr(), ws_n.value, _stream(stream)))
    return DeviceCSC(c.k, c.d_out, c.nnz, c.colptr, c.rowidx, codes8=codes, col_scale=scale,
                     code_kind=kind)


# ----------------------------------------------------------------- forward

def dict_workspace_size(n_layers: int, T: int, D: DeviceDict, Cs: DeviceCSC) -> int:
    n = C.c_size_t(0)
    d, c = D.desc(), Cs.desc()
    _check("dict_workspace_size",
           lib().dict_workspace_size(n_layers, T, C.byref(d), C.byref(c), C.byref(n)))
    return n.value


def workspace(n_layers: int, T: int, D: DeviceDict, Cs: DeviceCSC, device) -> torch.Tensor:
    """Forward workspace, zeroed: the library requires the whole workspace
    to be zero before its first use (the calls leave the control block and
    the tagged Z words zero again)."""
    return torch.zeros(dict_workspace_size(n_layers, T, D, Cs), dtype=torch.uint8, device=device)


def workspace_error_word(ws: torch.Tensor) -> int:
    """Word 32 of the control block: non-zero once a one-launch decode gave
    up waiting for a published Z word and computed it itself (a diagnostic:
    the results are still right)."""
    return int(ws[128:132].view(torch.int32).item())


def dict_group_forward(Xs, D: DeviceDict, Cs, Ys=None, ydtype=torch.float16, ws=None,
                       stream=None):
    """Y_l = (X_l D) C_l for every layer of a group sharing D."""
    n = len(Xs)
    T, d_in = Xs[0].shape
    d_out = Cs[0].d_out
    dev = Xs[0].device
    if Ys is None:
        Ys = [torch.empty(T, d_out, dtype=ydtype, device=dev) for _ in range(n)]
    _rows(Xs, "X", D.d_in)
    _rows(Ys, "Y", d_out)
    if len(Ys) != n or len(Cs) != n or Ys[0].shape[0] != T:
        raise ValueError("one X, one C and one Y of T rows per layer")
    if ws is None:
        ws = workspace(n, T, D, Cs[0], dev)
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in Xs])
    yp = (C.c_void_p * n)(*[y.data_ptr() for y in Ys])
    cs = (Csc * n)(*[c.desc() for c in Cs])
    d = D.desc()
    _check("dict_group_forward",
           lib().dict_group_forward(n, xp, _dt(Xs[0]), T, Xs[0].stride(0), C.byref(d), cs, yp,
                                    _dt(Ys[0]), Ys[0].stride(0), ws.data_ptr(), ws.numel(),
                                    _stream(stream)))
    return Ys


def dict_group_forward_noalloc(Xs, D: DeviceDict, Cs, Ys, stream=None):
    """dict_group_forward on the library's own workspace (no allocation in
    the call; Ys must be given)."""
    n = len(Xs)
    T = Xs[0].shape[0]
    _rows(Xs, "X", D.d_in)
    _rows(Ys, "Y", Cs[0].d_out)
    if len(Ys) != n or len(Cs) != n or Ys[0].shape[0] != T:
        raise ValueError("one X, one C and one Y of T rows per layer")
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in Xs])
    yp = (C.c_void_p * n)(*[y.data_ptr() for y in Ys])
    cs = (Csc * n)(*[c.desc() for c in Cs])
    d = D.desc()
    _check("dict_group_forward_noalloc",
           lib().dict_group_forward_noalloc(n, xp, _dt(Xs[0]), T, Xs[0].stride(0), C.byref(d), cs,
                                            yp, _dt(Ys[0]), Ys[0].stride(0), _stream(stream)))
    return Ys


def multi_workspace(n_dicts: int, n_layers: int, T: int, D: DeviceDict, Cs: DeviceCSC,
                    device) -> torch.Tensor:
    """Workspace of dict_multi_forward, zeroed (the library requires the
    whole workspace to be zero before its first use)."""
    n = C.c_size_t(0)
    d, c = D.desc(), Cs.desc()
    _check("dict_multi_workspace_size",
           lib().dict_multi_workspace_size(n_dicts, n_layers, T, C.byref(d), C.byref(c),
                                           C.byref(n)))
    return torch.zeros(n.value, dtype=torch.uint8, device=device)


def dict_multi_forward(Xs, Ds, Cs, Ys=None, ydtype=torch.float16, ws=None, stream=None):
    """Y[d * n + l] = (X_l D_d) C[d * n + l] for n = len(Xs) layers and the
    dictionaries Ds (q, k, v-like groups over the same activations); Cs is
    dictionary-major.  Returns the list of Y."""
    n, nd = len(Xs), len(Ds)
    assert len(Cs) == n * nd
    T = Xs[0].shape[0]
    dev = Xs[0].device
    if Ys is None:
        Ys = [torch.empty(T, Cs[0].d_out, dtype=ydtype, device=dev) for _ in range(n * nd)]
    _rows(Xs, "X", Ds[0].d_in)
    _rows(Ys, "Y", Cs[0].d_out)
    if len(Ys) != n * nd or Ys[0].shape[0] != T:
        raise ValueError("one Y of T rows per (dictionary, layer)")
    if ws is None:
        ws = multi_workspace(nd, n, T, Ds[0], Cs[0], dev)
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in Xs])
    yp = (C.c_void_p * (n * nd))(*[y.data_ptr() for y in Ys])
    ds = (Dict * nd)(*[D.desc() for D in Ds])
    cs = (Csc * (n * nd))(*[c.desc() for c in Cs])
    _check("dict_multi_forward",
           lib().dict_multi_forward(nd, n, xp, _dt(Xs[0]), T, Xs[0].stride(0), ds, cs, yp,
                                    _dt(Ys[0]), Ys[0].stride(0), ws.data_ptr(), ws.numel(),
                                    _stream(stream)))
    return Ys


def dict_proj_forward(X, D: DeviceDict, Cs: DeviceCSC, Y=None, ydtype=torch.float16, ws=None,
                      stream=None):
    T = X.shape[0]
    if Y is None:
        Y = torch.empty(T, Cs.d_out, dtype=ydtype, device=X.device)
    _rows([X], "X", D.d_in)
    _rows([Y], "Y", Cs.d_out)
    if Y.shape[0] != T:
        raise ValueError("Y needs the T rows of X")
    if ws is None:
        ws = workspace(1, T, D, Cs, X.device)
    d, c = D.desc(), Cs.desc()
    _check("dict_proj_forward",
           lib().dict_proj_forward(X.data_ptr(), _dt(X), T, X.stride(0), C.byref(d), C.byref(c),
                                   Y.data_ptr(), _dt(Y), Y.stride(0), ws.data_ptr(), ws.numel(),
                                   _stream(stream)))
    return Y


def dict_xd_forward(Xs, D: DeviceDict, zdtype=torch.float32, Z=None, ws=None, stream=None):
    n = len(Xs)
    T = Xs[0].shape[0]
    if Z is None:
        Z = torch.empty(n * T, D.k, dtype=zdtype, device=Xs[0].device)
    _rows(Xs, "X", D.d_in)
    if not Z.is_contiguous() or Z.shape != (n * T, D.k):
        raise ValueError(f"Z: a contiguous ({n * T}, {D.k}) tensor required")
    d = D.desc()
    need = C.c_size_t(0)
    _check("dict_xd_workspace_size",
           lib().dict_xd_workspace_size(n, T, C.byref(d), C.byref(need)))
    if ws is None and need.value:
        ws = torch.empty(need.value, dtype=torch.uint8, device=Xs[0].device)
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in Xs])
    _check("dict_xd_forward",
           lib().dict_xd_forward(n, xp, _dt(Xs[0]), T, Xs[0].stride(0), C.byref(d),
                                 Z.data_ptr(), _dt(Z), None if ws is None else ws.data_ptr(),
                                 0 if ws is None else ws.numel(), _stream(stream)))
    return Z


def dict_zc_forward(Z, T: int, Cs, Ys=None, ydtype=torch.float16, stream=None):
    n = len(Cs)
    d_out = Cs[0].d_out
    if Ys is None:
        Ys = [torch.empty(T, d_out, dtype=ydtype, device=Z.device) for _ in range(n)]
    _rows(Ys, "Y", d_out)
    if len(Ys) != n or Ys[0].shape[0] != T:
        raise ValueError("one Y of T rows per layer")
    if not Z.is_contiguous() or Z.shape != (n * T, Cs[0].k):
        raise ValueError(f"Z: a contiguous ({n * T}, {Cs[0].k}) tensor required")
    yp = (C.c_void_p * n)(*[y.data_ptr() for y in Ys])
    cs = (Csc * n)(*[c.desc() for c in Cs])
    _check("dict_zc_forward",
           lib().dict_zc_forward(n, Z.data_ptr(), _dt(Z), T, cs, yp, _dt(Ys[0]),
                                 Ys[0].stride(0), _stream(stream)))
    return Ys


# ----------------------------------------------------------------- producer steps

def dict_gram_inverse(D: DeviceDict, S: torch.Tensor, lam: float, stream=None):
    """P = (D^T S D + lam I)^-1 (k x k fp32).  Returns (P, error word): the
    error word is non-zero if the matrix was not positive definite."""
    assert S.dtype == torch.float32 and S.dim() == 2 and S.stride(1) == 1
    dev = S.device
    d = D.desc()
    n = C.c_size_t(0)
    _check("dict_gram_inverse_workspace_size",
           lib().dict_gram_inverse_workspace_size(C.byref(d), C.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
    P = torch.empty(D.k, D.k, dtype=torch.float32, device=dev)
    _check("dict_gram_inverse", lib().dict_gram_inverse(C.byref(d), S.data_ptr(), S.stride(0),
                                                        float(lam), P.data_ptr(), P.stride(0),
                                                        ws.data_ptr(), n.value, _stream(stream)))
    return P, ws[:4].view(torch.int32)


def dict_obs_prune(Cm: torch.Tensor, P: torch.Tensor, n_prune: int, stream=None):
    """Fixed-inverse pruning of every column of Cm (k x d_out fp32); returns
    (pruned coefficients fp32, keep mask uint8)."""
    assert Cm.dtype == torch.float32 and Cm.stride(1) == 1
    assert P.dtype == torch.float32 and P.stride(1) == 1
    k, d_out = Cm.shape
    out = torch.empty(k, d_out, dtype=torch.float32, device=Cm.device)
    keep = torch.empty(k, d_out, dtype=torch.uint8, device=Cm.device)
    _check("dict_obs_prune", lib().dict_obs_prune(k, d_out, Cm.data_ptr(), Cm.stride(0),
                                                  P.data_ptr(), P.stride(0), int(n_prune),
                                                  out.data_ptr(), out.stride(0), keep.data_ptr(),
                                                  keep.stride(0), _stream(stream)))
    return out, keep


def dict_refit(W: torch.Tensor, Cm: torch.Tensor, lam: float, stream=None):
    """Refit D (C C^T + lam I) = W C^T.  W: d_in x N, Cm: k x N (fp32).
    Returns (Dt: k x d_in fp32 atom-major, error word)."""
    assert W.dtype == torch.float32 and Cm.dtype == torch.float32
    assert W.stride(1) == 1 and Cm.stride(1) == 1
    d_in, N = W.shape
    k = Cm.shape[0]
    assert Cm.shape[1] == N
    n = C.c_size_t(0)
    _check("dict_refit_workspace_size", lib().dict_refit_workspace_size(d_in, k, C.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=W.device)
    Dt = torch.empty(k, d_in, dtype=torch.float32, device=W.device)
    _check("dict_refit", lib().dict_refit(d_in, N, k, W.data_ptr(), W.stride(0), Cm.data_ptr(),
                                          Cm.stride(0), float(lam), Dt.data_ptr(), Dt.stride(0),
                                          ws.data_ptr(), n.value, _stream(stream)))
    return Dt, ws[:4].view(torch.int32)


# ----------------------------------------------------------------- host -> device helpers

def to_device_dict(atoms_np, device, nvfp4: bool = False) -> DeviceDict:
    """Atom-major numpy dictionary (k, d_in) -> DeviceDict (NVFP4 via the
    library's own packer when ``nvfp4``)."""
    t = torch.from_numpy(atoms_np).to(device)
    k, d_in = atoms_np.shape
    if nvfp4:
        return DeviceDict(d_in, k, nv=nvfp4_pack(t.float().contiguous()))
    return DeviceDict.from_atoms(t)


def to_device_csc(dense_np, device, nvfp4: bool = False, fmt: str | None = None) -> DeviceCSC:
    """Dense numpy coefficients (k, d_out) -> DeviceCSC packed on the GPU.
    ``fmt``: None (the dense dtype, or NVFP4 when ``nvfp4``), "nvfp4", "fp8"
    or "int8" (values quantised by the library's own packers), or "block8"
    (block-structured support, blocks of 8 atoms)."""
    if fmt == "block8":
        return dict_pack_bcsc(torch.from_numpy(dense_np).to(device))
    c = dict_pack_csc(torch.from_numpy(dense_np).to(device))
    if fmt is None and nvfp4:
        fmt = "nvfp4"
    if fmt == "nvfp4":
        return csc_to_nvfp4(c)
    if fmt in CODE8:
        return csc_quantize8(c, fmt)
    return c


# ----------------------------------------------------------------- measurement support

def probe_mfma(blocks: int, iters: int, device="cuda:0", out=None, stream=None):
    """Matrix-core probe: blocks x 256 threads, each wave `iters` rounds of 8
    independent 32x32x16 f16 MFMAs on registers (blocks * 4 * iters * 8 *
    32768 FLOP).  Returns the per-thread outputs (blocks * 256 floats)."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    _check("dfs_probe_mfma", lib().dfs_probe_mfma(blocks, iters, out.data_ptr(), _stream(stream)))
    return out


def probe_mfma_flop(blocks: int, iters: int) -> float:
    return float(blocks) * 4 * iters * 8 * 32768


def probe_read(buf, blocks: int, out=None, stream=None):
    """HBM read probe: reads every byte of the device tensor `buf` once
    (blocks x 256 threads, grid-strided 16-byte words).  Returns the
    per-thread XORs (blocks * 256 uint32 as int32); their XOR is the XOR of
    every dword of buf."""
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    _check("dfs_probe_read", lib().dfs_probe_read(buf.data_ptr(), nbytes, blocks, out.data_ptr(),
                                                  _stream(stream)))
    return out
