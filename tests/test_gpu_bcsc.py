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


def _group(d_in, d_out, k, T, q, seed, dtype=np.float16):
    rng = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(rng.standard_normal((d_in, k)))
    Dt = np.ascontiguousarray((Q.T * 64 / np.sqrt(d_in)).astype(np.float16))
    Cs = [synth.block_coefficients(rng, k, d_out, q, dtype) for _ in range(2)]
    Xs = [rng.standard_normal((T, d_in)).astype(np.float16) for _ in range(2)]
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


def test_block_forward_above_16_rows_is_unsupported():
    say("case: block-structured forward with 2 x 9 rows")
    Dt, Cs, Xs = _group(256, 64, 64, 9, 0.5, 3)
    D = B.to_device_dict(Dt, DEV)
    Cg = [B.dict_pack_bcsc(torch.from_numpy(c).to(DEV)) for c in Cs]
    Xg = [torch.from_numpy(x).to(DEV) for x in Xs]
    with pytest.raises(B.DfsError) as ex:
        B.dict_group_forward(Xg, D, Cg)
    assert ex.value.status == 2


def test_equal_bytes_operands():
    # the block density that matches the headline 30% f16 CSC in bytes
    q = L.bcsc_density_at_equal_bytes(2048, 4096, int(0.3 * 2048 * 4096), "f16")
    assert abs(q - 0.5333) < 1e-3
