"""Seeded synthetic inputs shaped like the LLaMA-7B projections the pages study.

This module holds no arithmetic of the method: it only draws dictionaries,
coefficient matrices and activations with numpy, so that the HIP path and the
CPU oracle can be fed the same bytes.  It imports neither of them.

Recipes (one per workload; "density" is the kept fraction 1 - p):
  tiny          group of 2, d_in = d_out = 256, k = 128; D fp32 with orthonormal
                columns (reduced QR of an N(0,1) matrix); C fp32, each entry kept
                with probability 0.25, values N(0, 1/k); X 8 x 256 fp32 N(0,1).
  qproj         group of 2, d_in = d_out = 4096, k = 2048; D fp16 = orthonormal
                columns * 64/sqrt(d_in); C fp16 N(0, 1/k) at density 0.30; X fp16
                N(0,1), T = 1 (decode) or 2048 (prefill).
  mlp           group of 4; gate/up 4096 -> 11008, down 11008 -> 4096, k = 3072;
                D fp16 orthonormal * 64/sqrt(d_in) per type; C fp16 at density
                0.20; T = 1 or 16.
  stack_nvfp4   32 layers in groups of 2, 7 projection types (q, k, v, o: 4096 ->
                4096; gate, up: 4096 -> 11008; down: 11008 -> 4096), k =
                min(d_in, d_out) / 2; D fp32 N(0, 1/d_in) and C fp32 N(0, 1/k) at
                density 0.25, both later quantised to NVFP4; X fp16, T = 1.
Masks are independent Bernoulli draws per entry, so per-column nnz is binomial.
A kept value that rounds to zero in its storage dtype is redrawn, so the mask
equals the stored support.
Every tensor has its own seed: numpy ``SeedSequence([workload_id, group,
type_id, tensor_id])``, tensor_id 0 for D, 1 + 2l for C_l, 2 + 2l for X_l.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# The prefill workload is the decode group with 2048 tokens: same D and C.
WORKLOAD_IDS = {"tiny": 1, "qproj": 2, "qproj_prefill": 2, "mlp": 4, "stack_nvfp4": 5}

PROJ_TYPES = ("q", "k", "v", "o", "gate", "up", "down")


def llama7b_shape(ptype: str) -> tuple[int, int]:
    """(d_in, d_out) of a LLaMA-7B projection type."""
    if ptype in ("q", "k", "v", "o"):
        return 4096, 4096
    if ptype in ("gate", "up"):
        return 4096, 11008
    if ptype == "down":
        return 11008, 4096
    raise KeyError(ptype)


def rng_for(workload: str, group: int, type_id: int, tensor_id: int) -> np.random.Generator:
    ss = np.random.SeedSequence([WORKLOAD_IDS[workload], group, type_id, tensor_id])
    return np.random.default_rng(ss)


def dictionary(rng: np.random.Generator, d_in: int, k: int, rule: str, dtype) -> np.ndarray:
    """Atom-major dictionary: a (k, d_in) array whose row a is atom a
    (column a of the d_in x k matrix D_g).

    rule "orthonormal": reduced QR of an N(0,1) d_in x k matrix, columns
    scaled by 64/sqrt(d_in) (scale 1 for the tiny workload, see ``scale``).
    rule "gauss": N(0, 1/d_in) entries."""
    if rule.startswith("orthonormal"):
        scale = 1.0 if rule == "orthonormal" else 64.0 / np.sqrt(d_in)
        a = rng.standard_normal((d_in, k), dtype=np.float32)
        q, _ = np.linalg.qr(a)
        return np.ascontiguousarray((q * np.float32(scale)).T).astype(dtype)
    if rule == "gauss":
        a = rng.standard_normal((k, d_in), dtype=np.float32) * np.float32(1.0 / np.sqrt(d_in))
        return a.astype(dtype)
    raise KeyError(rule)


def coefficients(rng: np.random.Generator, k: int, d_out: int, density: float, dtype) -> np.ndarray:
    """Dense k x d_out coefficients: each entry kept with probability
    ``density`` (independently), kept values N(0, 1/k) stored in ``dtype`` and
    redrawn until nonzero in that dtype; the rest exactly 0."""
    mask = rng.random((k, d_out), dtype=np.float32) < np.float32(density)
    vals = (rng.standard_normal((k, d_out), dtype=np.float32)
            * np.float32(1.0 / np.sqrt(k))).astype(dtype)
    bad = mask & (vals == 0)
    while bad.any():
        redraw = (rng.standard_normal(int(bad.sum()), dtype=np.float32)
                  * np.float32(1.0 / np.sqrt(k))).astype(dtype)
        vals[bad] = redraw
        bad = mask & (vals == 0)
    out = np.zeros((k, d_out), dtype)
    out[mask] = vals[mask]
    return out


def activations(rng: np.random.Generator, T: int, d_in: int, dtype) -> np.ndarray:
    return rng.standard_normal((T, d_in), dtype=np.float32).astype(dtype)


@dataclass
class Group:
    """One layer group: a shared dictionary and per-layer C_l and X_l (dense,
    host numpy).  ``D`` is atom-major (k, d_in)."""
    workload: str
    ptype: str
    d_in: int
    d_out: int
    k: int
    T: int
    D: np.ndarray
    Cs: list = field(default_factory=list)
    Xs: list = field(default_factory=list)

    @property
    def n_layers(self) -> int:
        return len(self.Cs)


def block_coefficients(rng: np.random.Generator, k: int, d_out: int, block_density: float,
                       dtype) -> np.ndarray:
    """Dense k x d_out coefficients with block-structured support: each block
    of 8 consecutive rows of a column (the last may be shorter) is kept with
    probability ``block_density`` (independently); every entry of a kept
    block is N(0, 1/k) in ``dtype``, redrawn until nonzero; the rest is 0."""
    nb = (k + 7) // 8
    keep = rng.random((nb, d_out), dtype=np.float32) < np.float32(block_density)
    mask = np.repeat(keep, 8, axis=0)[:k]
    vals = (rng.standard_normal((k, d_out), dtype=np.float32)
            * np.float32(1.0 / np.sqrt(k))).astype(dtype)
    bad = mask & (vals == 0)
    while bad.any():
        vals[bad] = (rng.standard_normal(int(bad.sum()), dtype=np.float32)
                     * np.float32(1.0 / np.sqrt(k))).astype(dtype)
        bad = mask & (vals == 0)
    return np.where(mask, vals, np.zeros((), dtype)).astype(dtype)


def make_group(workload: str, *, group: int = 0, ptype: str = "q", T: int | None = None,
               n_layers: int | None = None, d_in: int | None = None, d_out: int | None = None,
               k: int | None = None, density: float | None = None,
               wdtype=None, xdtype=None) -> Group:
    """Draw one group of a named workload.  Keyword overrides allow the parity
    tests to draw smaller members of the same family (same recipe, other sizes)."""
    if workload == "tiny":
        spec = dict(n=2, d_in=256, d_out=256, k=128, density=0.25, T=8, rule="orthonormal",
                    wdt=np.float32, xdt=np.float32)
    elif workload in ("qproj", "qproj_prefill"):
        spec = dict(n=2, d_in=4096, d_out=4096, k=2048, density=0.30,
                    T=1 if workload == "qproj" else 2048, rule="orthonormal_scaled",
                    wdt=np.float16, xdt=np.float16)
    elif workload == "mlp":
        di, do = llama7b_shape(ptype)
        spec = dict(n=4, d_in=di, d_out=do, k=3072, density=0.20, T=1,
                    rule="orthonormal_scaled", wdt=np.float16, xdt=np.float16)
    elif workload == "stack_nvfp4":
        di, do = llama7b_shape(ptype)
        spec = dict(n=2, d_in=di, d_out=do, k=min(di, do) // 2, density=0.25, T=1, rule="gauss",
                    wdt=np.float32, xdt=np.float16)
    else:
        raise KeyError(workload)
    for key, val in (("n", n_layers), ("d_in", d_in), ("d_out", d_out), ("k", k),
                     ("density", density), ("T", T), ("wdt", wdtype), ("xdt", xdtype)):
        if val is not None:
            spec[key] = val
    type_id = PROJ_TYPES.index(ptype)
    D = dictionary(rng_for(workload, group, type_id, 0), spec["d_in"], spec["k"], spec["rule"],
                   spec["wdt"])
    g = Group(workload, ptype, spec["d_in"], spec["d_out"], spec["k"], spec["T"], D)
    for layer in range(spec["n"]):
        g.Cs.append(coefficients(rng_for(workload, group, type_id, 1 + 2 * layer), spec["k"],
                                 spec["d_out"], spec["density"], spec["wdt"]))
        g.Xs.append(activations(rng_for(workload, group, type_id, 2 + 2 * layer), spec["T"],
                                spec["d_in"], spec["xdt"]))
    return g
