"""Several dictionaries over the same activations (dict_multi_forward):
Y[d * n + l] = (X_l D_d) C[d * n + l], as the q, k and v projections of the
same layers compute (Eq. (1) per dictionary, Figure 2's one dictionary per
group).  At decode the whole set is one launch.  Each group must equal
dict_group_forward on that group bit for bit (the launch computes every Z
word and every output column with the same arithmetic, whichever workgroup
does it) and the oracle within the tolerance."""
import numpy as np
import pytest
import torch

from dictionary_factored_sparse_amd import binding as B, synth
from gpu_helpers import assert_close, device_group, oracle_group, say

pytestmark = pytest.mark.gpu

PTYPES = ("q", "k", "v", "o")


def _groups(nd, **kw):
    gs = [synth.make_group("qproj", ptype=p, **kw) for p in PTYPES[:nd]]
    for g in gs[1:]:
        g.Xs = gs[0].Xs  # one set of activations for every dictionary
    return gs


def _check(gs, dfmt, cfmt, reps=1):
    devs = [device_group(g, dfmt=dfmt, cfmt=cfmt) for g in gs]
    Xs = devs[0][2]
    Ds = [d[0] for d in devs]
    Cs = [c for d in devs for c in d[1]]
    n = len(Xs)
    ws = B.multi_workspace(len(Ds), n, Xs[0].shape[0], Ds[0], Cs[0], Xs[0].device)
    outs = []
    for _ in range(reps):  # repeated calls on one workspace
        outs.append([y.clone() for y in B.dict_multi_forward(Xs, Ds, Cs, ws=ws)])
    torch.cuda.synchronize()
    assert B.workspace_error_word(ws) == 0
    Ys = outs[-1]
    for o in outs[:-1]:
        for a, b in zip(o, Ys):
            assert torch.equal(a, b)
    for d, g in enumerate(gs):
        alone = B.dict_group_forward(Xs, Ds[d], devs[d][1])
        torch.cuda.synchronize()
        for l in range(n):
            assert torch.equal(Ys[d * n + l], alone[l]), (d, l)
        for l, ref in enumerate(oracle_group(g, dfmt=dfmt, cfmt=cfmt)):
            assert_close(Ys[d * n + l], ref, f"dictionary {d} layer {l}")


@pytest.mark.parametrize("nd", [2, 3])
@pytest.mark.parametrize("fmt", [("plain", "plain"), ("nvfp4", "nvfp4"), ("nvfp4", "plain")])
def test_multi_decode_full_size(nd, fmt):
    # 4096 -> 4096, k = 2048, two layers: with 3 dictionaries each wave takes
    # 3 atoms, so some waves straddle two dictionaries
    say(f"case: {nd} dictionaries, q_proj shape, D {fmt[0]}, C {fmt[1]}, T=1")
    _check(_groups(nd), *fmt, reps=2)


@pytest.mark.parametrize("nd,n_layers", [(2, 1), (3, 1), (3, 2)])
def test_multi_decode_ragged(nd, n_layers):
    say(f"case: {nd} dictionaries, d_in=512, d_out=300, k=200, {n_layers} layer(s)")
    _check(_groups(nd, d_in=512, d_out=300, k=200, n_layers=n_layers), "plain", "plain")


def test_multi_runs_group_by_group_elsewhere():
    # four dictionaries, and three tokens: the groups run in turn
    say("case: 4 dictionaries at T=1, and 3 dictionaries at T=3 (group by group)")
    _check(_groups(4, d_in=512, d_out=300, k=200), "plain", "plain")
    _check(_groups(3, d_in=512, d_out=300, k=200, T=3), "plain", "plain")
