"""GPU tests of flex_attn_bwd_noalloc, the backward for callers that cannot
allocate: called through the C ABI, its gradients equal flex_attn_bwd's
(given its own workspace) bit for bit, on two calls in a row, the second on a
smaller problem (the scratch keeps the first call's contents, which the
second must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_grad_inputs, make_inputs, workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _both(cfg):
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=True)
    qd, kd, vd, dod, dld = (t.to(DEV) for t in (q, k, v, dout, dlse))
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"], return_lse=True)
    ref = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg.get("score"), cfg["scale"], dlse=dld,
                 grad_dtype=torch.float32)
    got = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg.get("score"), cfg["scale"], dlse=dld,
                 grad_dtype=torch.float32, noalloc=True)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    (("prefix_causal", dict(B=2, H=4, q_len=1000, kv_len=1000,
                            mask={"kind": "prefix_causal", "prefix": 300})),
     ("sliding_window", dict(B=1, H=2, q_len=333, kv_len=333))),
    (("causal_rel_bias", dict(B=1, H=8, q_len=700, kv_len=700)),
     ("long_causal_d128", dict(B=1, H=2, q_len=200, kv_len=200))),
    # fp32 inputs (the vector-ALU kernels), value head dims unlike the key's
    (("prefix_causal", dict(B=1, H=2, q_len=520, kv_len=520, dtype="fp32", dv=128,
                            mask={"kind": "prefix_causal", "prefix": 200})),
     ("long_causal_d128", dict(B=1, H=1, q_len=150, kv_len=150, dtype="fp32", dv=64))),
])
def test_noalloc_backward_equals_workspace_backward(first, second):
    for name, over in (first, second):
        ref, got = _both(workload(name, **over))
        for a, b, g in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(a, b), "%s %s differs" % (name, g)
            assert torch.isfinite(a).all()


def test_noalloc_backward_rejects_beyond_its_scratch():
    """2 B H q_len above the scratch size: FLEX_E_SCRATCH_LIMIT, nothing
    launched (checked before any device call)."""
    lib = fa.load()
    rows = fa.NOALLOC_SCRATCH_FLOATS // 2 + 1
    bm = fa.BlockMaskStruct()
    bmt = fa.BlockMaskTStruct()
    code = lib.flex_attn_bwd_noalloc(None, None, None, None, None, None, None, 0, 1, 1, rows,
                                     rows, 64, 64, ctypes.byref(bm), ctypes.byref(bmt), None,
                                     0.125, None, None, None, 0, None)
    assert code == fa.FLEX_E_SCRATCH_LIMIT
    assert "scratch" in fa.strerror(code)
