"""The matrix-core probe behind the prefill GEMM's measured peak.

Its operands make every product exact: B is all ones and A holds quarters,
so each 32x32x16 MFMA adds the same block, whose entries sum to
32 * (sum of A over the wave) = 32 * 192 = 6144.  With 8 accumulators per
wave and 4 waves per workgroup, a workgroup's 256 outputs sum to
196608 per round whatever the operand layout, and with the documented
layout (lane l holds row l % 32, K elements 8 * (l / 32) .. + 7) every
thread holds 768 per round.
"""
import pytest
import torch

from dictionary_factored_sparse_amd import binding as B
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters", [1, 3, 64])
def test_probe_mfma_runs_every_round(iters):
    say(f"case: MFMA probe, 6 workgroups, {iters} rounds")
    out = B.probe_mfma(6, iters).view(6, 256)
    torch.cuda.synchronize()
    assert torch.equal(out.double().sum(dim=1),
                       torch.full((6,), 196608.0 * iters, dtype=torch.float64, device=out.device))
    assert torch.equal(out, torch.full_like(out, 768.0 * iters))


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 3), (1 << 20, 64), ((1 << 20) + 48, 7)])
def test_probe_read_reads_every_word(nbytes, blocks):
    # the XOR of the per-thread outputs is the XOR of every dword of the
    # buffer, so a word the probe skipped or read twice shows
    say(f"case: read probe, {nbytes} bytes, {blocks} workgroups")
    g = torch.Generator().manual_seed(nbytes + blocks)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int64, generator=g)
    host = host.to(torch.int32)
    buf = host.to("cuda:0")
    out = B.probe_read(buf, blocks)
    torch.cuda.synchronize()
    got = 0
    for v in out.cpu().numpy().view("uint32").tolist():
        got ^= v
    want = 0
    for v in host.numpy().view("uint32").tolist():
        want ^= v
    assert got == want
