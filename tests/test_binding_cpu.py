"""CPU-only checks that the Python binding refuses, before any library call
that could launch a kernel, tensors the kernels cannot reach: host tensors,
block-mask arrays of the wrong dtype or size, and block masks built for other
lengths."""
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa


def _cpu_mask(q_len=256, kv_len=256, qb=128, kb=64):
    nq, nk = fa.block_mask_dims(q_len, kv_len, qb, kb)
    z = lambda *s: torch.zeros(s, dtype=torch.int32)
    return fa.BlockMask({"kind": "causal"}, q_len, kv_len, qb, kb, z(nq), z(nq, nk), z(nq),
                        z(nq, nk))


@pytest.mark.parametrize("build", [fa.build_block_mask, fa.build_block_mask_t])
def test_block_mask_build_refuses_host_device(build):
    with pytest.raises(ValueError):
        build({"kind": "causal"}, 256, 256, 128, 64, device="cpu")


def test_block_mask_build_refuses_host_arrays():
    with pytest.raises(ValueError):
        fa.build_block_mask({"kind": "causal"}, 256, 256, 128, 64, out=_cpu_mask())


def test_block_mask_build_refuses_mismatched_out():
    with pytest.raises(ValueError):
        fa.build_block_mask({"kind": "causal"}, 512, 256, 128, 64, out=_cpu_mask())


def test_fwd_refuses_host_tensors():
    q = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, _cpu_mask())


def test_bwd_refuses_host_tensors():
    q = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 256)
    bmt = fa.BlockMaskT({"kind": "causal"}, 256, 256, 128, 64,
                        *[torch.zeros(s, dtype=torch.int32) for s in ((4,), (4, 2), (4,), (4, 2))])
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, q, lse, _cpu_mask(), bmt)
