"""Seeded random sweep of the backward (dq, dk, dv) against the fp64 oracle:
mask kind and parameters, score modification, head dims, tile shape, ragged
and unequal lengths, gradient dtype and the log-sum-exp gradient are drawn
per case; the bar is the one in test_bwd_gpu.py.  (Document masks have
their own backward cases in test_document_gpu.py.)"""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_grad_inputs, make_inputs, workload
from test_bwd_gpu import check, oracle_bwd, run_bwd

pytestmark = pytest.mark.gpu

HEAD_DIMS = [(64, 64), (128, 128), (64, 128), (128, 64)]
TILES = [(64, 64), (128, 64), (128, 128)]


def _case(seed):
    r = np.random.default_rng(8000 + seed)
    d, dv = HEAD_DIMS[r.integers(len(HEAD_DIMS))]
    qb, kb = TILES[r.integers(len(TILES))]
    kind = ["noop", "causal", "sliding_window", "prefix_causal"][r.integers(4)]
    lq, lk = int(r.integers(1, 500)), int(r.integers(1, 500))
    if kind == "sliding_window":
        mask = {"kind": kind, "window": int(r.integers(0, 300)), "window_min": int(r.integers(0, 3))}
    elif kind == "prefix_causal":
        mask = {"kind": kind, "prefix": int(r.integers(0, lq))}
    else:
        mask = {"kind": kind}
    score = {"kind": "rel_bias", "bias_max": 8.0} if r.integers(3) == 0 else {"kind": "identity"}
    over = dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), q_len=lq, kv_len=lk, d=d, dv=dv,
                q_block=qb, kv_block=kb, mask=mask, score=score, seed=9500 + seed)
    grad_dtype = torch.bfloat16 if r.integers(2) else torch.float32
    return over, grad_dtype, bool(r.integers(3) == 0)


@pytest.mark.parametrize("seed", range(32))
def test_random_case(seed):
    over, grad_dtype, with_dlse = _case(seed)
    cfg = workload("prefix_causal", **over)
    cfg["scale"] = fa.default_scale(cfg["d"])
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=with_dlse)
    got = run_bwd(cfg, q, k, v, dout, dlse, grad_dtype)
    ref = oracle_bwd(cfg, q, k, v, dout, dlse)
    check(got, ref, grad_dtype, "seed %d: %s" % (seed, over))
