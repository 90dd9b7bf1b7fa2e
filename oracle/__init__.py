"""CPU oracle for the factored dictionary projection (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library: it loads ``oracle/liboracle.so`` (built from ``oracle/oracle.c`` by
``oracle/build.py``) and marshals numpy arrays.

Pages (cited by title and section):
  Review: "DictLLM: Shared Dictionaries for Post-Training Compression".

* ``forward`` -- Eq. (1) of the Review ("Prerequisites: projections, rank and
  calibration"): Z = X D, Y = Z C, float64, sums in ascending index order.
* ``pack_csc`` -- support-keeping export of C (Review, Algorithm 2: export of
  dictionary, codes, scales and support; zeros preserved as absent).
* ``nvfp4_pack``/``nvfp4_unpack`` -- 4-bit E2M1 values with one 8-bit E4M3
  scale per 16 values (Review, "From retained values to measured decoding")
  and one fp32 tensor scale.  The scale recipe is a reading; parity unpinned
  against the pages, pinned against format definitions and bounds.
* ``pack_bcsc``/``forward_bcsc`` -- block-structured support, blocks of 8
  consecutive atoms per column (Review, "Let the accelerator constrain the
  support").
* ``gram_inverse``, ``obs_delete``, ``obs_prune``, ``refit`` -- the producer
  steps of the Review ("Method II: prune in coefficient space", Eq. (6)-(7)
  and Algorithm 1; "Method III: refit the dictionary", Eq. (9)).
* ``quantize8_csc`` -- 8-bit coefficient codes, FP8 (E4M3) or INT8, for the
  mixed-precision rows of Table 4 on the tables page ("DictLLM: Post-training
  Compression of Large Language Model with Dictionary Kernels").  Reading:
  one fp32 scale per column of C, amax / 448 or amax / 127, nearest code with
  ties to even (the pages leave the scaling open).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DFS_ORACLE_LIB selects another build of oracle.c (the sanitizer build)
_LIB_PATH = os.environ.get("DFS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

DT_F32, DT_F16, DT_NVFP4, DT_FP8, DT_INT8 = 0, 1, 2, 3, 4   # element types of oracle.c


class _Tensor(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("data", C.c_void_p), ("codes", C.c_void_p),
                ("scales", C.c_void_p), ("ts", C.c_float), ("col_scale", C.c_void_p)]


_lib = None


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.orc_half_value.restype = C.c_double
        L.orc_half_value.argtypes = [C.c_uint16]
        L.orc_e2m1_value.restype = C.c_double
        L.orc_e2m1_value.argtypes = [C.c_int]
        L.orc_e4m3_value.restype = C.c_double
        L.orc_e4m3_value.argtypes = [C.c_int]
        L.orc_e4m3_nearest.restype = C.c_int
        L.orc_e4m3_nearest.argtypes = [C.c_float]
        L.orc_e2m1_nearest.restype = C.c_int
        L.orc_e2m1_nearest.argtypes = [C.c_float]
        L.orc_nvfp4_tensor_scale.restype = C.c_float
        L.orc_nvfp4_tensor_scale.argtypes = [C.c_float]
        L.orc_nvfp4_pack.restype = C.c_int
        L.orc_nvfp4_pack.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                     C.POINTER(C.c_float)]
        L.orc_nvfp4_unpack.restype = None
        L.orc_nvfp4_unpack.argtypes = [C.c_void_p, C.c_void_p, C.c_float, C.c_int64,
                                       C.c_void_p]
        L.orc_int8_nearest.restype = C.c_int
        L.orc_int8_nearest.argtypes = [C.c_float]
        L.orc_quant8_csc.restype = C.c_int
        L.orc_quant8_csc.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32,
                                     C.c_void_p, C.c_void_p]
        L.orc_pack_csc.restype = C.c_int64
        L.orc_pack_csc.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64]
        L.orc_forward.restype = C.c_int
        L.orc_forward.argtypes = [C.c_int32, C.POINTER(_Tensor), C.c_int64, C.c_int32,
                                  C.c_int32, C.POINTER(_Tensor), C.c_int64, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.POINTER(_Tensor), C.c_void_p]
        L.orc_pack_bcsc.restype = C.c_int64
        L.orc_pack_bcsc.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64]
        L.orc_forward_bcsc.restype = C.c_int
        L.orc_forward_bcsc.argtypes = [C.c_int32, C.POINTER(_Tensor), C.c_int64, C.c_int32,
                                       C.c_int32, C.POINTER(_Tensor), C.c_int64, C.c_int32,
                                       C.c_void_p, C.c_void_p, C.POINTER(_Tensor), C.c_void_p]
        L.orc_gram_inverse.restype = C.c_int
        L.orc_gram_inverse.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_double,
                                       C.c_void_p]
        L.orc_obs_delete.restype = C.c_double
        L.orc_obs_delete.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_int32]
        L.orc_obs_prune.restype = C.c_int
        L.orc_obs_prune.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                                    C.c_void_p, C.c_void_p]
        L.orc_refit.restype = C.c_int
        L.orc_refit.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                C.c_double, C.c_void_p]
        L.orc_max_threads.restype = C.c_int
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- formats

def half_value(bits: int) -> float:
    return lib().orc_half_value(int(bits))


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e4m3_nearest(s: float) -> int:
    return lib().orc_e4m3_nearest(float(np.float32(s)))


def e2m1_nearest(v: float) -> int:
    return lib().orc_e2m1_nearest(float(np.float32(v)))


def int8_nearest(v: float) -> int:
    return lib().orc_int8_nearest(float(np.float32(v)))


def nvfp4_tensor_scale(amax: float) -> float:
    return lib().orc_nvfp4_tensor_scale(float(np.float32(amax)))


@dataclass
class NVFP4:
    """An NVFP4 tensor of ``n`` elements: packed codes, block scales, ts."""
    codes: np.ndarray   # uint8[(n+1)//2], element 2i in the low nibble
    scales: np.ndarray  # uint8[(n+15)//16], E4M3 codes
    ts: float           # fp32 tensor scale
    n: int


def nvfp4_pack(x: np.ndarray) -> NVFP4:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    scales = np.zeros((n + 15) // 16, np.uint8)
    ts = C.c_float(0.0)
    rc = lib().orc_nvfp4_pack(_ptr(x), n, _ptr(codes), _ptr(scales), C.byref(ts))
    if rc != 0:
        raise ValueError("nvfp4_pack: input holds NaN or Inf")
    return NVFP4(codes, scales, float(ts.value), n)


def nvfp4_unpack(q: NVFP4) -> np.ndarray:
    y = np.empty(q.n, np.float32)
    lib().orc_nvfp4_unpack(_ptr(q.codes), _ptr(q.scales), q.ts, q.n, _ptr(y))
    return y


@dataclass
class Codes8:
    """8-bit coefficient values in CSC order with one fp32 scale per column:
    entry p of column j decodes to value(codes[p]) * col_scale[j]."""
    kind: str               # "fp8" (E4M3) or "int8"
    codes: np.ndarray       # uint8[nnz]
    col_scale: np.ndarray   # float32[d_out]

    @property
    def dtype_code(self) -> int:
        return DT_FP8 if self.kind == "fp8" else DT_INT8


# ---------------------------------------------------------------- CSC

@dataclass
class CSC:
    """k x d_out coefficient matrix, column-compressed.

    ``vals`` is a float16/float32 array (bit copies of the dense entries) or
    an ``NVFP4`` holding the values in CSC order."""
    k: int
    d_out: int
    colptr: np.ndarray  # int32[d_out+1]
    rowidx: np.ndarray  # uint16[nnz]
    vals: object

    @property
    def nnz(self) -> int:
        return int(self.colptr[-1])


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.float16:
        return DT_F16
    raise TypeError(f"unsupported dtype {a.dtype}")


def pack_csc(Cd: np.ndarray) -> CSC:
    """Dense row-major k x d_out (float16/float32) -> canonical CSC."""
    Cd = np.ascontiguousarray(Cd)
    k, d_out = Cd.shape
    dt = _dtype_code(Cd)
    colptr = np.zeros(d_out + 1, np.int32)
    nnz = lib().orc_pack_csc(_ptr(Cd), dt, k, d_out, d_out, _ptr(colptr), None, None, 0)
    rowidx = np.zeros(max(nnz, 1), np.uint16)
    vals = np.zeros(max(nnz, 1), Cd.dtype)
    got = lib().orc_pack_csc(_ptr(Cd), dt, k, d_out, d_out, _ptr(colptr), _ptr(rowidx),
                             _ptr(vals), nnz)
    assert got == nnz
    return CSC(k, d_out, colptr, rowidx[:nnz], vals[:nnz])


def quantize8_csc(c: CSC, kind: str) -> CSC:
    """Quantise a CSC's float16/float32 values to 8-bit codes, ``kind``
    "fp8" (E4M3) or "int8", one scale per column; support unchanged."""
    if kind not in ("fp8", "int8"):
        raise ValueError(kind)
    vals = np.ascontiguousarray(c.vals)
    colptr = np.ascontiguousarray(c.colptr, np.int32)
    codes = np.zeros(max(c.nnz, 1), np.uint8)
    scale = np.zeros(max(c.d_out, 1), np.float32)
    q = Codes8(kind, codes, scale)
    if vals.size == 0:
        vals = np.zeros(1, np.float32)
    rc = lib().orc_quant8_csc(_ptr(vals), _dtype_code(vals), _ptr(colptr), c.d_out,
                              q.dtype_code, _ptr(codes), _ptr(scale))
    if rc != 0:
        raise ValueError("quantize8_csc: values hold NaN or Inf")
    return CSC(c.k, c.d_out, c.colptr, c.rowidx, Codes8(kind, codes[:c.nnz], scale[:c.d_out]))


def csc_to_nvfp4(c: CSC) -> CSC:
    """Quantise a CSC's values (in CSC order) to NVFP4; support unchanged."""
    return CSC(c.k, c.d_out, c.colptr, c.rowidx,
               nvfp4_pack(np.asarray(c.vals, np.float32)))


# ---------------------------------------------------------------- forward

def _tensor(t, keep: list) -> _Tensor:
    if isinstance(t, NVFP4):
        keep.extend([t.codes, t.scales])
        return _Tensor(DT_NVFP4, None, _ptr(t.codes), _ptr(t.scales), t.ts, None)
    if isinstance(t, Codes8):
        codes = t.codes if t.codes.size else np.zeros(1, np.uint8)
        keep.extend([codes, t.col_scale])
        return _Tensor(t.dtype_code, _ptr(codes), None, None, 0.0, _ptr(t.col_scale))
    a = np.ascontiguousarray(t)
    keep.append(a)
    return _Tensor(_dtype_code(a), _ptr(a), None, None, 0.0, None)


def forward(X: np.ndarray, D, d_in: int, c: CSC) -> np.ndarray:
    """Y = (X D) C in float64.

    X: T x d_in (float16/float32).  D: the dictionary stored atom by atom,
    i.e. a k x d_in array (row a is atom a) or an ``NVFP4`` of the k*d_in
    elements in that order.  c: ``CSC``.  Returns T x d_out float64."""
    X = np.ascontiguousarray(X)
    T = X.shape[0]
    assert X.shape[1] == d_in
    keep: list = []
    tx = _tensor(X, keep)
    td = _tensor(D, keep)
    tc = _tensor(c.vals, keep)
    colptr = np.ascontiguousarray(c.colptr, np.int32)
    rowidx = np.ascontiguousarray(c.rowidx, np.uint16)
    if rowidx.size == 0:
        rowidx = np.zeros(1, np.uint16)
    Y = np.zeros((T, c.d_out), np.float64)
    rc = lib().orc_forward(T, C.byref(tx), d_in, d_in, c.k, C.byref(td), d_in, c.d_out,
                           _ptr(colptr), _ptr(rowidx), C.byref(tc), _ptr(Y))
    if rc == -2:
        raise ValueError("oracle forward: not a CSC (colptr or a row index out of range)")
    if rc != 0:
        raise MemoryError("oracle forward: allocation failed")
    return Y


def group_forward(Xs, D, d_in: int, cs) -> list:
    """The group's layers share D; each layer has its own X_l and C_l
    (Review, Figure 2: shared weights with separate activations)."""
    return [forward(X, D, d_in, c) for X, c in zip(Xs, cs)]


# ---------------------------------------------------------------- block-structured support

@dataclass
class BCSC:
    """k x d_out coefficients kept in blocks of 8 consecutive atoms: kept
    block q of column j has block index bidx[q] (rows 8*bidx[q] .. +7) and
    values vals[8q .. 8q+7]."""
    k: int
    d_out: int
    colptr: np.ndarray  # int32[d_out+1], counts blocks
    bidx: np.ndarray    # uint16[nblk]
    vals: np.ndarray    # float16/float32[8 * nblk]

    @property
    def nblk(self) -> int:
        return int(self.colptr[-1])


def pack_bcsc(Cd: np.ndarray) -> BCSC:
    """Dense row-major k x d_out (float16/float32) -> block-structured CSC."""
    Cd = np.ascontiguousarray(Cd)
    k, d_out = Cd.shape
    dt = _dtype_code(Cd)
    colptr = np.zeros(d_out + 1, np.int32)
    n = lib().orc_pack_bcsc(_ptr(Cd), dt, k, d_out, d_out, _ptr(colptr), None, None, 0)
    bidx = np.zeros(max(n, 1), np.uint16)
    vals = np.zeros(8 * max(n, 1), Cd.dtype)
    got = lib().orc_pack_bcsc(_ptr(Cd), dt, k, d_out, d_out, _ptr(colptr), _ptr(bidx),
                              _ptr(vals), n)
    assert got == n
    return BCSC(k, d_out, colptr, bidx[:n], vals[:8 * n])


def forward_bcsc(X: np.ndarray, D, d_in: int, b: BCSC) -> np.ndarray:
    """Y = (X D) C with block-structured C, float64 (zeros inside kept
    blocks included)."""
    X = np.ascontiguousarray(X)
    T = X.shape[0]
    keep: list = []
    tx = _tensor(X, keep)
    td = _tensor(D, keep)
    vals = b.vals if b.vals.size else np.zeros(8, np.float32)
    tc = _tensor(vals, keep)
    colptr = np.ascontiguousarray(b.colptr, np.int32)
    bidx = np.ascontiguousarray(b.bidx, np.uint16)
    if bidx.size == 0:
        bidx = np.zeros(1, np.uint16)
    Y = np.zeros((T, b.d_out), np.float64)
    rc = lib().orc_forward_bcsc(T, C.byref(tx), d_in, d_in, b.k, C.byref(td), d_in, b.d_out,
                                _ptr(colptr), _ptr(bidx), C.byref(tc), _ptr(Y))
    if rc == -2:
        raise ValueError("oracle forward_bcsc: not a block CSC (colptr or a block index out of range)")
    if rc != 0:
        raise MemoryError("oracle forward_bcsc: allocation failed")
    return Y


# ---------------------------------------------------------------- producer steps

def gram_inverse(Dt: np.ndarray, S: np.ndarray, lam: float) -> np.ndarray:
    """P = (D^T S D + lam I)^-1 (Review Eq. (6)-(7)).  Dt: k x d_in (atom
    a is row a), S: d_in x d_in; both taken as fp32.  Returns float64 k x k."""
    Dt = np.ascontiguousarray(Dt, np.float32)
    S = np.ascontiguousarray(S, np.float32)
    k, d_in = Dt.shape
    P = np.zeros((k, k), np.float64)
    rc = lib().orc_gram_inverse(d_in, k, _ptr(Dt), _ptr(S), float(lam), _ptr(P))
    if rc != 0:
        raise ValueError("gram_inverse: matrix not positive definite")
    return P


def obs_delete(P: np.ndarray, c: np.ndarray, i: int):
    """One Eq. (7) deletion of coordinate i with compensation: returns the
    moved vector and the saliency c_i^2 / P_ii."""
    P = np.ascontiguousarray(P, np.float64)
    c = np.array(c, np.float64)
    s = lib().orc_obs_delete(P.shape[0], _ptr(P), _ptr(c), int(i))
    return c, s


def obs_prune(C: np.ndarray, P: np.ndarray, n_prune: int):
    """Fixed-inverse pruning of every column of C (k x d_out, fp32) with the
    fixed inverse P (k x k, fp32), n_prune rows per column (Review Algorithm
    1).  Returns (float64 pruned C, uint8 keep mask)."""
    C = np.ascontiguousarray(C, np.float32)
    P = np.ascontiguousarray(P, np.float32)
    k, d_out = C.shape
    out = np.zeros((k, d_out), np.float64)
    keep = np.zeros((k, d_out), np.uint8)
    rc = lib().orc_obs_prune(k, d_out, _ptr(C), _ptr(P), int(n_prune), _ptr(out), _ptr(keep))
    if rc != 0:
        raise ValueError("obs_prune: non-positive P_ii or allocation failure")
    return out, keep


def refit(W: np.ndarray, Cm: np.ndarray, lam: float) -> np.ndarray:
    """Dictionary refit, Review Eq. (9): D (C C^T + lam I) = W C^T.  W: d_in x N,
    Cm: k x N (pruned coefficients of the group's layers side by side), both
    fp32.  Returns D atom by atom (k x d_in, row a = atom a), float64."""
    W = np.ascontiguousarray(W, np.float32)
    Cm = np.ascontiguousarray(Cm, np.float32)
    d_in, N = W.shape
    k = Cm.shape[0]
    Dt = np.zeros((k, d_in), np.float64)
    rc = lib().orc_refit(d_in, N, k, _ptr(W), _ptr(Cm), float(lam), _ptr(Dt))
    if rc != 0:
        raise ValueError("refit: Gram matrix not positive definite")
    return Dt


def max_threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))
