"""dict_group_forward_noalloc (the group forward on the library's own
workspace, for callers that cannot allocate) against dict_group_forward,
through the C ABI, on calls in a row with shrinking inputs on the one shared
array: the one-launch decode of the q_proj group, then a smaller decode
group, a stacked-row (MFMA + SpMM) group, and a tiny fp32 group.  Bar: max
|Y_noalloc - Y| <= 2e-3 max |Y| against the existing entry point, and the
oracle's bound on the same inputs."""
import numpy as np
import pytest
import torch

from dictionary_factored_sparse_amd import binding as B
from dictionary_factored_sparse_amd import synth
from tests.gpu_helpers import assert_close, device_group, oracle_group, say

pytestmark = pytest.mark.gpu


def _check(g, **fmt):
    D, Cs, Xs = device_group(g, **fmt)
    ref = B.dict_group_forward(Xs, D, Cs, ydtype=torch.float32)
    Ys = [torch.full_like(y, float("nan")) for y in ref]
    B.dict_group_forward_noalloc(Xs, D, Cs, Ys)
    torch.cuda.synchronize()
    for l, oref in enumerate(oracle_group(g, **fmt)):
        assert_close(Ys[l], ref[l].double().cpu().numpy(), f"vs dict_group_forward, layer {l}")
        assert_close(Ys[l], oref, f"vs oracle, layer {l}")


def test_noalloc_matches_group_forward_on_shrinking_calls():
    cases = [
        ("q_proj decode group, 2 x 4096 -> 4096, k = 2048", synth.make_group("qproj"), {}),
        ("smaller decode group, k = 512", synth.make_group("qproj", d_in=1024, d_out=768, k=512,
                                                           T=1, n_layers=2), {}),
        ("stacked rows, 2 x T = 40 (MFMA, SpMM)",
         synth.make_group("qproj", d_in=1024, d_out=776, k=512, T=40, n_layers=2), {}),
        ("NVFP4 factors, smaller decode", synth.make_group("stack_nvfp4", ptype="q", d_in=512,
                                                           d_out=384, k=256), {"nvfp4": True}),
        ("tiny fp32 group, 8 tokens", synth.make_group("tiny"), {}),
    ]
    for what, g, fmt in cases:
        say(f"case: no-allocation entry point, {what}")
        _check(g, **fmt)
