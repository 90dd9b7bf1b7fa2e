"""The workspace contract of the one-launch decode (Eq. (1) at T = 1, Z handed
between workgroups as tagged words in the workspace), on the GPU:

* when a workgroup's bounded wait for a published Z word gives up, it computes
  the word itself from X and D_g, so Y still matches the oracle; the host
  forces that path by setting the poll bound to 0, which makes every
  workgroup compute every word it needs without polling (every kernel runs
  to its end: nothing waits without a bound);
* the control block holds only a diagnostic word (the epochs of the Z hand-off
  live in the tagged region after it), so a caller that re-zeroes the control
  block (or nothing) between calls on one workspace gets right results;
* fp32 activations and dictionaries above 16 stacked rows run with the
  workspace size the query returns.

Bound: max|Y_gpu - Y_ref| <= 2e-3 * max|Y_ref|."""
import os

import numpy as np
import pytest
import torch

from dictionary_factored_sparse_amd import binding as B
from dictionary_factored_sparse_amd import synth
from tests.gpu_helpers import DEV, assert_close, device_group, oracle_group, say

pytestmark = pytest.mark.gpu

CTRL = 4096


class _spin_limit:
    """Sets DFS_SPIN_LIMIT for the calls inside the block (read per call)."""

    def __init__(self, n):
        self.n = str(n)

    def __enter__(self):
        os.environ["DFS_SPIN_LIMIT"] = self.n

    def __exit__(self, *exc):
        os.environ.pop("DFS_SPIN_LIMIT", None)


@pytest.mark.parametrize("wl,ptype,n,dfmt,cfmt", [
    ("qproj", "q", 2, "plain", "plain"),       # the headline group
    ("mlp", "down", 4, "plain", "fp8"),        # d_in = 11008: three X passes per row
    ("stack_nvfp4", "q", 2, "nvfp4", "nvfp4"),
])
def test_decode_computes_z_itself_when_waits_give_up(wl, ptype, n, dfmt, cfmt):
    say(f"case: one-launch decode with poll bound 0, {wl} {ptype} n={n} D {dfmt} C {cfmt}")
    g = synth.make_group(wl, ptype=ptype, n_layers=n, T=1)
    D, Cs, Xs = device_group(g, dfmt=dfmt, cfmt=cfmt)
    ws = B.workspace(n, 1, D, Cs[0], DEV)
    ref_run = B.dict_group_forward(Xs, D, Cs, ws=ws)
    torch.cuda.synchronize()
    assert B.workspace_error_word(ws) == 0
    with _spin_limit(0):
        Ys = B.dict_group_forward(Xs, D, Cs, ws=ws)
        torch.cuda.synchronize()
    # no poll: every workgroup computed its Z words itself and said so
    assert B.workspace_error_word(ws) == 1
    refs = oracle_group(g, dfmt=dfmt, cfmt=cfmt)
    for l, ref in enumerate(refs):
        assert_close(Ys[l], ref, f"bound 0, layer {l}")
        assert_close(ref_run[l], ref, f"normal, layer {l}")
    # the diagnostic word stays set until the caller clears it; later calls
    # with the normal bound are unaffected
    ws[128:132].zero_()
    again = B.dict_group_forward(Xs, D, Cs, ws=ws)
    torch.cuda.synchronize()
    assert B.workspace_error_word(ws) == 0
    for a, b in zip(again, ref_run):
        assert torch.equal(a, b)


def test_multi_dictionary_decode_computes_z_itself():
    say("case: three dictionaries in one launch (NVFP4 stack q, k, v) with poll bound 0")
    gs = [synth.make_group("stack_nvfp4", ptype=p, T=1) for p in ("q", "k", "v")]
    for g in gs[1:]:
        g.Xs = gs[0].Xs
    devs = [device_group(g, nvfp4=True) for g in gs]
    Xs = devs[0][2]
    Ds = [d[0] for d in devs]
    Cs = [c for d in devs for c in d[1]]
    ws = B.multi_workspace(3, 2, 1, Ds[0], Cs[0], DEV)
    with _spin_limit(0):
        Ys = B.dict_multi_forward(Xs, Ds, Cs, ws=ws)
        torch.cuda.synchronize()
    assert B.workspace_error_word(ws) == 1
    for d, g in enumerate(gs):
        for l, ref in enumerate(oracle_group(g, nvfp4=True)):
            assert_close(Ys[d * 2 + l], ref, f"dictionary {d} layer {l}")


def test_control_block_rezeroed_between_calls():
    # Two calls on one workspace with different activations: first with
    # nothing cleared between them, then with only the control block
    # re-zeroed.  The epochs that tag the Z words live after the control
    # block, so no call can take a word the previous one published.
    say("case: one workspace, different X per call, control block re-zeroed or not")
    g = synth.make_group("qproj", d_in=2048, d_out=3000, k=1024, T=1, n_layers=2)
    g2 = synth.make_group("qproj", d_in=2048, d_out=3000, k=1024, T=1, n_layers=2, group=5)
    g2.D, g2.Cs = g.D, g.Cs  # same factors, other activations
    D, Cs, Xa = device_group(g)
    Xb = [torch.from_numpy(X).to(DEV) for X in g2.Xs]
    ra, rb = oracle_group(g), oracle_group(g2)
    ws = B.workspace(2, 1, D, Cs[0], DEV)
    for it, (Xs, refs) in enumerate(((Xa, ra), (Xb, rb), (Xa, ra), (Xb, rb), (Xa, ra))):
        if it >= 2:
            ws[:CTRL].zero_()
        Ys = B.dict_group_forward(Xs, D, Cs, ws=ws)
        torch.cuda.synchronize()
        assert B.workspace_error_word(ws) == 0
        assert int(ws[:CTRL].count_nonzero()) == 0
        for l, ref in enumerate(refs):
            assert_close(Ys[l], ref, f"call {it} layer {l}")


@pytest.mark.parametrize("xdt,wdt", [(np.float32, np.float32), (np.float32, np.float16),
                                     (np.float16, np.float32)])
def test_fp32_above_16_rows_with_the_queried_workspace(xdt, wdt):
    # 2 layers x 32 tokens = 64 stacked rows: dot-product Z (fp32) and the
    # token-tiled SpMM; the binding sizes the workspace with the query
    say(f"case: tiny group, 2 x T=32, X {np.dtype(xdt).name}, D/C {np.dtype(wdt).name}")
    g = synth.make_group("tiny", T=32, wdtype=wdt, xdtype=xdt)
    D, Cs, Xs = device_group(g)
    ws = B.workspace(2, 32, D, Cs[0], DEV)
    Ys = B.dict_group_forward(Xs, D, Cs, ws=ws, ydtype=torch.float32)
    torch.cuda.synchronize()
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"layer {l}")


@pytest.mark.parametrize("d_in,k,T", [(256, 128, 32), (2048, 2048, 16), (2048, 2048, 40)])
def test_fp32_z_keeps_its_range(d_in, k, T):
    # fp32 activations scaled so that |Z| runs far above the f16 range
    # (65504): every path keeps fp32 Z unrounded, in fp32 LDS tiles (T > 16,
    # and T = 16 at k = 2048 where an f16 tile would otherwise be chosen)
    say(f"case: fp32 group, |Z| > 65504, d_in={d_in} k={k} T={T}")
    g = synth.make_group("tiny", d_in=d_in, k=k, T=T)
    g.Xs = [np.ascontiguousarray(X * np.float32(1e5)) for X in g.Xs]
    D, Cs, Xs = device_group(g)
    ws = B.workspace(2, T, D, Cs[0], DEV)
    Ys = B.dict_group_forward(Xs, D, Cs, ws=ws, ydtype=torch.float32)
    torch.cuda.synchronize()
    zmax = max(float(np.abs(X.astype(np.float64) @ g.D.astype(np.float64).T).max()) for X in g.Xs)
    assert zmax > 65504.0
    for l, ref in enumerate(oracle_group(g)):
        assert_close(Ys[l], ref, f"layer {l}")


def test_two_decodes_on_two_streams():
    # two one-launch decodes of the MLP gate group (about 82 KiB of LDS per
    # workgroup: one workgroup per CU) issued on two streams, so that their
    # grids may share the CUs and neither be resident whole.  A workgroup
    # whose wait gives up (bound: 2000 polls, a few milliseconds) computes its
    # Z words itself; every result matches the oracle either way.
    say("case: two MLP gate decodes on two streams, poll bound 2000, 8 rounds")
    gs = [synth.make_group("mlp", ptype="gate", group=g, T=1) for g in (0, 1)]
    devs = [device_group(g) for g in gs]
    wss = [B.workspace(4, 1, d[0], d[1][0], DEV) for d in devs]
    refs = [oracle_group(g) for g in gs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    rounds = 8
    Ys = [[[torch.empty(1, gs[0].d_out, dtype=torch.float16, device=DEV) for _ in range(4)]
           for _ in range(2)] for _ in range(rounds)]
    torch.cuda.synchronize()
    with _spin_limit(2000):
        for r in range(rounds):
            for i in range(2):
                D, Cs, Xs = devs[i]
                B.dict_group_forward(Xs, D, Cs, Ys=Ys[r][i], ws=wss[i], stream=streams[i])
        torch.cuda.synchronize()
    say("diagnostic words: " + str([B.workspace_error_word(w) for w in wss]))
    for r in range(rounds):
        for i in range(2):
            for l in range(4):
                assert_close(Ys[r][i][l], refs[i][l], f"round {r} stream {i} layer {l}")
