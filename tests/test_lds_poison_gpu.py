"""The LDS-poison debugging mode of the bf16 forward (environment variable
FLEXATTN_DEBUG_LDS_POISON): each K/V staging buffer is filled with NaN
before its next loads are issued.  With the kernel's waits and barriers in
place the results must be bit-identical to the normal run and free of NaN;
a missing wait would read the NaN fill.  Cases cover every mask kind, both
head dims, a value head dim other than the key's, every tile shape, ragged
tails, subtiling and the exact running max."""
import os

import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_inputs, with_doc_ids, workload
from parity import compare, oracle_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ENV = "FLEXATTN_DEBUG_LDS_POISON"

CASES = [
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000,
                           mask={"kind": "prefix_causal", "prefix": 300}), {}),
    ("sliding_window", dict(B=1, H=2, q_len=1100, kv_len=1100), {}),
    ("sliding_window", dict(B=1, H=2, q_len=1100, kv_len=1100), dict(use_subtiling=True)),
    ("long_causal_d128", dict(B=1, H=2, q_len=777, kv_len=777), {}),
    ("causal_rel_bias", dict(B=1, H=4, q_len=700, kv_len=700, q_block=64, kv_block=64), {}),
    ("document_causal", dict(B=1, H=2, q_len=900, kv_len=900, doc_len_min=1, doc_len_max=300), {}),
    ("prefix_causal", dict(B=1, H=2, q_len=300, kv_len=650, mask={"kind": "noop"}, d=64, dv=128),
     {}),
    ("prefix_causal", dict(B=1, H=2, q_len=650, kv_len=333, mask={"kind": "causal"}), dict(max=True)),
]


def _run(q, k, v, bm, cfg, poison, use_subtiling=False, want_max=False):
    old = os.environ.pop(ENV, None)
    try:
        if poison:
            os.environ[ENV] = "1"
        res = fa.fwd(q, k, v, bm, cfg.get("score"), cfg["scale"], out_dtype=torch.float32,
                     return_lse=True, use_subtiling=use_subtiling, return_max=want_max)
        torch.cuda.synchronize()
    finally:
        os.environ.pop(ENV, None)
        if old is not None:
            os.environ[ENV] = old
    return [t.cpu() for t in res]


@pytest.mark.parametrize("name,over,opt", CASES, ids=[f"{n}-{i}" for i, (n, _o, _p) in enumerate(CASES)])
def test_poisoned_run_is_bitwise_normal(name, over, opt):
    cfg = workload(name, **over)
    mask = with_doc_ids(cfg)
    q, k, v = make_inputs(cfg)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    dm = dict(mask, q_doc=mask["q_doc"].to(DEV), kv_doc=mask["kv_doc"].to(DEV)) \
        if "q_doc" in mask else mask
    bm = fa.build_block_mask(dm, cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"],
                             device=DEV)
    kw = dict(use_subtiling=opt.get("use_subtiling", False), want_max=opt.get("max", False))
    print("case", name, over, opt, flush=True)
    normal = _run(qd, kd, vd, bm, cfg, False, **kw)
    poisoned = _run(qd, kd, vd, bm, cfg, True, **kw)
    for a, b in zip(normal, poisoned):
        assert not torch.isnan(b).any()
        assert torch.equal(a, b)
    # and the poisoned run against the oracle, as every forward
    ref_out, ref_lse = oracle_rows(dict(cfg, mask=mask), q, k, v)
    out, lse = poisoned[0].double().numpy(), poisoned[1].double().numpy()
    compare(out.reshape(-1, out.shape[-1]), lse.reshape(-1), ref_out, ref_lse, cfg["dtype"],
            "fp32", what=name + " (poisoned LDS)")
