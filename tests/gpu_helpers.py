"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, run the oracle on the same inputs, and
compare to the bound max|Y_gpu - Y_ref| <= 2e-3 * max|Y_ref| (0 when the
reference is identically 0)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from dictionary_factored_sparse_amd import binding as B

TOL = 2e-3
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(y_gpu: torch.Tensor, y_ref: np.ndarray, what: str):
    y = y_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), what
    ref_max = float(np.abs(y_ref).max()) if y_ref.size else 0.0
    err = float(np.abs(y - y_ref).max()) if y_ref.size else 0.0
    if ref_max == 0.0:
        assert err == 0.0, f"{what}: reference is 0, gpu max |y| = {err}"
    else:
        assert err <= TOL * ref_max, f"{what}: max err {err:.3e} > {TOL} * {ref_max:.3e}"
    return err, ref_max


def _fmts(nvfp4, dfmt, cfmt):
    """Storage of (D, C): "plain" (the synth dtype) or "nvfp4"; C may also be
    "fp8" or "int8" (8-bit codes, one scale per column); `nvfp4` sets both."""
    base = "nvfp4" if nvfp4 else "plain"
    return dfmt or base, cfmt or base


def device_group(g, nvfp4: bool = False, dfmt=None, cfmt=None):
    """Upload a synth.Group: D (atom-major), packed C_l, X_l."""
    dfmt, cfmt = _fmts(nvfp4, dfmt, cfmt)
    D = B.to_device_dict(g.D, DEV, nvfp4=dfmt == "nvfp4")
    Cs = [B.to_device_csc(Cd, DEV, fmt=None if cfmt == "plain" else cfmt) for Cd in g.Cs]
    Xs = [torch.from_numpy(X).to(DEV) for X in g.Xs]
    return D, Cs, Xs


def oracle_group(g, nvfp4: bool = False, rows=None, dfmt=None, cfmt=None):
    """Oracle outputs for every layer (optionally for a subset of tokens);
    quantised factors enter as the oracle's own quantisation of the same
    values."""
    dfmt, cfmt = _fmts(nvfp4, dfmt, cfmt)
    D = O.nvfp4_pack(g.D.astype(np.float32)) if dfmt == "nvfp4" else g.D
    if cfmt == "nvfp4":
        cs = [O.csc_to_nvfp4(O.pack_csc(Cd.astype(np.float32))) for Cd in g.Cs]
    elif cfmt in ("fp8", "int8"):
        cs = [O.quantize8_csc(O.pack_csc(Cd), cfmt) for Cd in g.Cs]
    else:
        cs = [O.pack_csc(Cd) for Cd in g.Cs]
    Xs = g.Xs if rows is None else [X[rows] for X in g.Xs]
    return O.group_forward(Xs, D, g.d_in, cs)
