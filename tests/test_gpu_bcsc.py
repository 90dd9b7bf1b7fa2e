"""GPU parity of the block-structured support variant (blocks of 8
consecutive atoms per column; "DictLLM: Shared Dictionaries for Post-Training
Compression", "Let the accelerator constrain the support") against the
oracle, through the C ABI: the packer bit-exactly, the forward within
2e-3 * max|Y_ref|."""
import numpy as np
import pytest
import torch

import oracle as O
from dictionary_factored_sparse_amd import binding as B
from dictionary_factored_sparse_amd import ledger as L
from dictionary_factored_sparse_amd import synth
from tests.gpu_helpers import DEV, assert_close, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k,d_out,dtype,structured", [(2048, 4096, np.float16, True),
                                                      (70, 33, np.float32, True),
                                                      (128, 256, np.float16, False),
                                                      (8, 1, np.float16, True),
                                                      (64, 64, np.float32, False)])
def test_pack_bcsc_bit_exact(k, d_out, dtype, structured):
    say(f"case: dict_pack_bcsc k={k} d_out={d_out} {np.dtype(dtype).name} structured={structured}")
    rng = np.random.default_rng(k + d_out)
    if structured:
        Cd = synth.block_coefficients(rng, k, d_out, 0.5, dtype)
    else:
        Cd = synth.coefficients(rng, k, d_out, 0.1, dtype)
    c = B.dict_pack_bcsc(torch.from_numpy(Cd).to(DEV))
    torch.cuda.synchronize()
    ref = O.pack_bcsc(Cd)
    assert c.nnz == ref.nblk
    assert np.array_equal(c.colptr.cpu().numpy(), ref.colptr)
    assert np.array_equal(c.rowidx[:c.nnz].cpu().numpy().view(np.uint16), ref.bidx)
    assert np.array_equal(c.vals[:8 * c.nnz].cpu().numpy().view(np.uint8), ref.vals.view(np.uint8))


def _group(d_in, d_out, k, T, q, seed, dtype=np.float16, n_layers=2):
    rng = np.random.default_rng(seed)
    if k <= d_in:
        Q, _ = np.linalg.qr(rng.standard_normal((d_in, k)))
        Dt = (Q.T * 64 / np.sqrt(d_in)).astype(dtype)
    else:  # more atoms than d_in: Gaussian atoms of the same scale
        Dt = (rng.standard_normal((k, d_in)) * 64 / d_in).astype(dtype)
    Dt = np.ascontiguousarray(Dt)
    Cs = [synth.block_coefficients(rng, k, d_out, q, dtype) for _ in range(n_layers)]
    xdt = np.float16 if dtype == np.float16 else np.float32
    Xs = [rng.standard_normal((T, d_in)).astype(xdt) for _ in range(n_layers)]
    return Dt, Cs, Xs


@pytest.mark.parametrize("d_in,d_out,k,T", [(512, 400, 256, 1), (512, 400, 256, 3),
                                            (512, 400, 72, 5), (2048, 512, 2048, 16),
                                            (4096, 4096, 2048, 1)])
def test_block_forward(d_in, d_out, k, T):
    say(f"case: block-structured forward d_in={d_in} d_out={d_out} k={k} T={T}")
    q = 0.533  # the fraction of blocks an unstructured 30% f16 CSC buys at equal bytes
    Dt, Cs, Xs = _group(d_in, d_out, k, T, q, d_in + k + T)
    D = B.to_device_dict(Dt, DEV)
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to(DEV)) for c in Cs]
    Xg = [torch.from_numpy(x).to(DEV) for x in Xs]
    # a group stacks 2T rows (at most 16 on this path); T = 16 runs one layer
    # at a time, two token tiles of 8 at k = 2048
    if 2 * T <= 16:
        Ys = B.dict_group_forward(Xg, D, Cg)
    else:
        Ys = [B.dict_proj_forward(Xg[l], D, Cg[l]) for l in range(2)]
    torch.cuda.synchronize()
    for l in range(2):
        ref = O.forward_bcsc(Xs[l], Dt, d_in, O.pack_bcsc(Cs[l]))
        assert_close(Ys[l], ref, f"block layer {l}")
    Y1 = B.dict_proj_forward(Xg[1], D, Cg[1])
    torch.cuda.synchronize()
    assert torch.equal(Y1, Ys[1])


def _both_decode_paths(Xg, D, Cg):
    import os
    out = {}
    for path in ("fused", "two"):
        if path == "two":
            os.environ["DFS_DECODE_PATH"] = "two"
        try:
            out[path] = B.dict_group_forward(Xg, D, Cg)
            torch.cuda.synchronize()
        finally:
            os.environ.pop("DFS_DECODE_PATH", None)
    return out


@pytest.mark.parametrize("d_in,d_out,k,n", [(4096, 4096, 2048, 2), (512, 400, 256, 2),
                                            (1024, 1000, 512, 4), (11008, 4096, 3072, 2),
                                            (512, 33, 72, 1)])
def test_block_one_launch_decode(d_in, d_out, k, n):
    # T = 1: one launch (X D, Z hand-off, blocks of 8 contiguous Z words per
    # kept block) against the oracle and against the two-launch path
    say(f"case: block-structured one-launch decode d_in={d_in} d_out={d_out} k={k} n={n}")
    Dt, Cs, Xs = _group(d_in, d_out, k, 1, 0.533, d_in + k + n, n_layers=n)
    D = B.to_device_dict(Dt, DEV)
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to(DEV)) for c in Cs]
    Xg = [torch.from_numpy(x).to(DEV) for x in Xs]
    out = _both_decode_paths(Xg, D, Cg)
    for l in range(n):
        ref = O.forward_bcsc(Xs[l], Dt, d_in, O.pack_bcsc(Cs[l]))
        assert_close(out["fused"][l], ref, f"one-launch layer {l}")
        assert_close(out["two"][l], ref, f"two-launch layer {l}")


@pytest.mark.parametrize("d_in,d_out,k,T,dtype", [(512, 400, 256, 9, np.float16),
                                                  (512, 400, 256, 40, np.float16),
                                                  (1024, 776, 520, 100, np.float16),
                                                  (512, 300, 2048, 33, np.float16),
                                                  (256, 64, 72, 17, np.float32),
                                                  (2048, 512, 6000, 20, np.float16),
                                                  (256, 100, 70, 20, np.float16),
                                                  (256, 96, 16384, 20, np.float16)])
def test_block_spmm_above_16_rows(d_in, d_out, k, T, dtype):
    # 2 x T stacked rows > 16: MFMA X D (f16 Z; VALU fp32 Z for f32 factors),
    # then the block SpMM over token tiles of up to 32 (ragged last tile;
    # k = 6000 stages an 8-token tile and k = 16384 a 4-token one; k = 70
    # ends in a block that reaches past k, whose atoms from k on are zero in
    # the staged tile)
    say(f"case: block-structured prefill d_in={d_in} d_out={d_out} k={k} T={T}")
    Dt, Cs, Xs = _group(d_in, d_out, k, T, 0.533, d_in + k + T, dtype=dtype)
    D = B.to_device_dict(Dt, DEV)
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to(DEV)) for c in Cs]
    Xg = [torch.from_numpy(x).to(DEV) for x in Xs]
    Ys = B.dict_group_forward(Xg, D, Cg, ydtype=torch.float32)
    torch.cuda.synchronize()
    for l in range(2):
        ref = O.forward_bcsc(Xs[l], Dt, d_in, O.pack_bcsc(Cs[l]))
        assert_close(Ys[l], ref, f"block prefill layer {l}")


def test_block_prefill_q_proj_group():
    # the q_proj group's shape at equal bytes (53.3% of 8-atom blocks kept),
    # 2 x 2048 tokens, sampled tokens against the oracle
    say("case: block-structured prefill, 2 x 4096 -> 4096, k = 2048, T = 2048 (sampled tokens)")
    Dt, Cs, Xs = _group(4096, 4096, 2048, 2048, 0.533, 11)
    D = B.to_device_dict(Dt, DEV)
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to(DEV)) for c in Cs]
    Xg = [torch.from_numpy(x).to(DEV) for x in Xs]
    Ys = B.dict_group_forward(Xg, D, Cg)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 33, 511, 1023, 1024, 2015, 2047])
    for l in range(2):
        ref = O.forward_bcsc(Xs[l][rows], Dt, 4096, O.pack_bcsc(Cs[l]))
        assert_close(Ys[l][torch.from_numpy(rows).to(DEV)], ref, f"q_proj block prefill layer {l}")


def test_equal_bytes_operands():
    # the block density that matches the headline 30% f16 CSC in bytes
    q = L.bcsc_density_at_equal_bytes(2048, 4096, int(0.3 * 2048 * 4096), "f16")
    assert abs(q - 0.5333) < 1e-3
