"""GPU forward with a value head dim different from the query / key head dim
(the V_HEAD_DIM of the pages' kernel template, "[Inductor][Flex Attention]
Add Subtiling Option for Alpha Scaling", flex_attention.py hunks) vs the fp64
oracle, which takes Dv as its own argument.  Bars as for the other forward
tests: bf16 inputs out 1e-2 (fp32 output; bf16 output adds half a bf16 ulp),
lse 1e-3; fp32 inputs the fp32 bar of tests/parity.py on out and lse."""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_inputs, with_doc_ids, workload
from oracle import oracle
from parity import compare, sample_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _run(cfg, rows=None, out_dtype="fp32", **kw):
    q, k, v = make_inputs(cfg)
    assert v.shape[-1] == cfg["dv"] and q.shape[-1] == cfg["d"]
    mask = with_doc_ids(cfg)
    dmask = with_doc_ids(cfg, DEV)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    bm = fa.build_block_mask(dmask, cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"],
                             device=DEV)
    od = {"fp32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    res = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"], out_dtype=od, return_lse=True, **kw)
    torch.cuda.synchronize()
    out, lse = res[0], res[1]
    Dv = cfg["dv"]
    assert out.shape[-1] == Dv
    o = out.double().cpu().numpy().reshape(-1, Dv)
    l = lse.double().cpu().numpy().reshape(-1)
    f = lambda t: t.float().numpy()
    ref = oracle.attention_rows(f(q), f(k), f(v), mask, cfg.get("score", {"kind": "identity"}),
                                cfg["scale"], rows=rows, with_max=len(res) == 3)
    if rows is not None:
        o, l = o[rows], l[rows]
    compare(o, l, ref[0], ref[1], cfg["dtype"], out_dtype, what="dv %d/%d" % (cfg["d"], Dv))
    if len(res) == 3:
        mx = res[2].double().cpu().numpy().reshape(-1)
        mx = mx[rows] if rows is not None else mx
        dead = np.isneginf(ref[2])
        assert np.array_equal(np.isneginf(mx), dead)
        assert np.abs(mx[~dead] - ref[2][~dead]).max() <= 1e-3


CASES = [
    (64, 128, 128, 64, dict(mask={"kind": "prefix_causal", "prefix": 300})),
    (64, 128, 64, 64, dict(mask={"kind": "causal"})),
    (64, 128, 128, 128, dict(mask={"kind": "sliding_window", "window": 200, "window_min": 3})),
    (128, 64, 128, 128, dict(mask={"kind": "causal"})),
    (128, 64, 128, 64, dict(mask={"kind": "noop"}, kv_len=650)),
    (128, 64, 64, 64, dict(mask={"kind": "document_causal"}, doc_len_min=20, doc_len_max=300)),
    (64, 128, 128, 128, dict(mask={"kind": "causal"}, score={"kind": "rel_bias", "bias_max": 8.0}, H=4)),
]


@pytest.mark.parametrize("d,dv,qb,kb,over", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-{i}" for i, c in enumerate(CASES)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_parity(d, dv, qb, kb, over, out_dtype):
    base = dict(B=1, H=2, q_len=777, kv_len=777, d=d, dv=dv, q_block=qb, kv_block=kb,
                score={"kind": "identity"})
    base.update(over)
    cfg = workload("prefix_causal", **base)
    cfg["scale"] = fa.default_scale(d)
    print("case", d, dv, qb, kb, over, out_dtype, flush=True)
    _run(cfg, out_dtype=out_dtype)


def test_options_with_dv():
    cfg = workload("prefix_causal", B=1, H=2, q_len=500, kv_len=500, d=64, dv=128)
    _run(cfg, return_max=True)
    _run(cfg, use_subtiling=True)


def test_full_size_sampled():
    """The prefix workload's shape with a 128-wide value head, sampled rows."""
    cfg = workload("prefix_causal", dv=128)
    _run(cfg, rows=sample_rows(cfg))


FP32_CASES = [
    (64, 128, 64, 64, dict(mask={"kind": "prefix_causal", "prefix": 300})),
    (64, 128, 128, 64, dict(mask={"kind": "sliding_window", "window": 200, "window_min": 3})),
    (64, 128, 128, 128, dict(mask={"kind": "causal"}, score={"kind": "rel_bias", "bias_max": 8.0}, H=4)),
    (128, 64, 64, 64, dict(mask={"kind": "document_causal"}, doc_len_min=20, doc_len_max=300)),
    (128, 64, 128, 64, dict(mask={"kind": "noop"}, kv_len=650)),
    (128, 64, 128, 128, dict(mask={"kind": "causal"}, q_len=333, kv_len=333)),
]


@pytest.mark.parametrize("d,dv,qb,kb,over", FP32_CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-{i}" for i, c in enumerate(FP32_CASES)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_fp32_parity(d, dv, qb, kb, over, out_dtype):
    """fp32 inputs with a value head dim unlike the key head dim."""
    base = dict(B=1, H=2, q_len=777, kv_len=777, d=d, dv=dv, q_block=qb, kv_block=kb,
                score={"kind": "identity"})
    base.update(over)
    cfg = workload("prefix_causal", **base)
    cfg["dtype"] = "fp32"
    cfg["scale"] = fa.default_scale(d)
    print("case fp32", d, dv, qb, kb, over, out_dtype, flush=True)
    _run(cfg, out_dtype=out_dtype)
