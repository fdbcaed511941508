"""GPU document masks (per-token document ids, optionally causal) vs the fp64
oracle, through the C ABI: block arrays bit-exact in both layouts, forward
and backward under the same bars as the other masks (forward: out 1e-2 with
fp32 output, lse 1e-3, fp32 inputs 1e-4; backward: 1e-2 of each gradient's
max magnitude + 1e-5).  Ids are non-decreasing, as the library requires."""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import (make_grad_inputs, make_inputs, with_doc_ids,
                                                          workload)
from oracle import oracle
from parity import compare, sample_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _ids(lengths):
    return torch.from_numpy(np.repeat(np.arange(len(lengths)), lengths).astype(np.int32))


def _mask(kind, q_doc, kv_doc=None):
    kv_doc = q_doc if kv_doc is None else kv_doc
    return {"kind": kind, "q_doc": q_doc, "kv_doc": kv_doc}


def _dev(mask):
    return dict(mask, q_doc=mask["q_doc"].to(DEV), kv_doc=mask["kv_doc"].to(DEV))


BUILD_CASES = [
    ([5, 1, 9, 3, 14, 64, 70, 2], 16, 16),
    ([130, 1, 500, 64, 64, 200], 64, 64),
    ([130, 1, 500, 64, 64, 200], 128, 64),
    ([1000], 128, 128),
    ([1] * 300, 32, 16),
]


@pytest.mark.parametrize("lengths,qb,kb", BUILD_CASES)
@pytest.mark.parametrize("kind", ["document", "document_causal"])
def test_block_arrays_match_oracle(lengths, qb, kb, kind):
    ids = _ids(lengths)
    L = int(ids.numel())
    mask = _mask(kind, ids)
    bm = fa.build_block_mask(_dev(mask), L, L, qb, kb, device=DEV)
    bmt = fa.build_block_mask_t(_dev(mask), L, L, qb, kb, device=DEV)
    torch.cuda.synchronize()
    for got, ref in ((bm.arrays(), oracle.block_mask(mask, L, L, qb, kb)),
                     (bmt.arrays(), oracle.block_mask_t(mask, L, L, qb, kb))):
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g.cpu().numpy(), r)


def test_block_arrays_cross_lengths():
    """Queries and keys with their own ids and lengths; ids 1 and 4 have no
    keys, id 3 no queries."""
    q_doc = torch.tensor([0] * 70 + [1] * 30 + [2] * 90 + [4] * 11, dtype=torch.int32)
    kv_doc = torch.tensor([0] * 20 + [2] * 150 + [3] * 77, dtype=torch.int32)
    Lq, Lk = q_doc.numel(), kv_doc.numel()
    for kind in ("document", "document_causal"):
        mask = _mask(kind, q_doc, kv_doc)
        for qb, kb in ((64, 64), (128, 64)):
            bm = fa.build_block_mask(_dev(mask), Lq, Lk, qb, kb, device=DEV)
            bmt = fa.build_block_mask_t(_dev(mask), Lq, Lk, qb, kb, device=DEV)
            torch.cuda.synchronize()
            for got, ref in ((bm.arrays(), oracle.block_mask(mask, Lq, Lk, qb, kb)),
                             (bmt.arrays(), oracle.block_mask_t(mask, Lq, Lk, qb, kb))):
                for g, r in zip(got, ref):
                    np.testing.assert_array_equal(g.cpu().numpy(), r)


def _fwd_case(cfg, mask, out_dtype="fp32"):
    q, k, v = make_inputs(cfg)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    bm = fa.build_block_mask(_dev(mask), cfg["q_len"], cfg["kv_len"], cfg["q_block"],
                             cfg["kv_block"], device=DEV)
    od = {"fp32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    out, lse = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"], out_dtype=od,
                      return_lse=True)
    torch.cuda.synchronize()
    f = lambda t: t.float().numpy()
    ref_out, ref_lse = oracle.attention_rows(f(q), f(k), f(v), mask, cfg.get("score", {"kind": "identity"}),
                                             cfg["scale"])
    D = cfg["d"]
    return compare(out.double().cpu().numpy().reshape(-1, D), lse.double().cpu().numpy().reshape(-1),
                   ref_out, ref_lse, cfg["dtype"], out_dtype, what=str(cfg["mask"]["kind"]))


FWD_CASES = [
    ("document_causal", dict(B=1, H=2, q_len=1000, kv_len=1000, doc_len_min=1, doc_len_max=300), {}),
    ("document_causal", dict(B=2, H=1, q_len=777, kv_len=777, doc_len_min=50, doc_len_max=400,
                             q_block=128, kv_block=64), {}),
    ("document_causal", dict(B=1, H=2, q_len=600, kv_len=600, q_block=64, kv_block=64,
                             mask={"kind": "document"}, doc_len_min=1, doc_len_max=250), {}),
    ("document_causal", dict(B=1, H=2, q_len=500, kv_len=500, d=128, doc_len_min=30, doc_len_max=200), {}),
    ("document_causal", dict(B=1, H=4, q_len=500, kv_len=500, score={"kind": "rel_bias", "bias_max": 8.0},
                             doc_len_min=20, doc_len_max=300), {}),
    ("document_causal", dict(B=1, H=1, q_len=300, kv_len=300, dtype="fp32", q_block=64, kv_block=64,
                             doc_len_min=1, doc_len_max=90), {}),
]


@pytest.mark.parametrize("name,over,_", FWD_CASES, ids=[f"{n}-{i}" for i, (n, _o, _x) in enumerate(FWD_CASES)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_forward_parity(name, over, _, out_dtype):
    cfg = workload(name, **over)
    cfg["scale"] = fa.default_scale(cfg["d"])
    mask = with_doc_ids(cfg)
    print("case", over, out_dtype, flush=True)
    _fwd_case(cfg, mask, out_dtype)


def test_forward_cross_lengths_and_empty_rows():
    """Query ids without keys give out 0 and lse -inf."""
    q_doc = torch.tensor([0] * 70 + [1] * 30 + [2] * 90 + [4] * 11, dtype=torch.int32)
    kv_doc = torch.tensor([0] * 20 + [2] * 150 + [3] * 77, dtype=torch.int32)
    for kind in ("document", "document_causal"):
        cfg = workload("document_causal", B=1, H=2, q_len=q_doc.numel(), kv_len=kv_doc.numel(),
                       q_block=64, kv_block=64)
        _fwd_case(cfg, _mask(kind, q_doc, kv_doc))


def test_forward_full_size_sampled():
    """The packed-document workload at full size, sampled rows."""
    cfg = workload("document_causal")
    mask = with_doc_ids(cfg)
    q, k, v = make_inputs(cfg)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    bm = fa.build_block_mask(_dev(mask), cfg["q_len"], cfg["kv_len"], cfg["q_block"],
                             cfg["kv_block"], device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], out_dtype=torch.float32,
                      return_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(cfg)
    # also the first and last rows of every document
    ids = mask["q_doc"].numpy()
    starts = np.flatnonzero(np.r_[1, np.diff(ids)])
    ends = np.r_[starts[1:] - 1, len(ids) - 1]
    rows = np.unique(np.r_[rows, starts, ends]).astype(np.int64)
    f = lambda t: t.float().numpy()
    ref_out, ref_lse = oracle.attention_rows(f(q), f(k), f(v), mask, cfg["score"], cfg["scale"],
                                             rows=rows)
    compare(out.double().cpu().numpy().reshape(-1, 64)[rows], lse.double().cpu().numpy().reshape(-1)[rows],
            ref_out, ref_lse, "bf16", "fp32", what="full document")


@pytest.mark.parametrize("over", [
    dict(B=1, H=2, q_len=700, kv_len=700, doc_len_min=1, doc_len_max=260),
    dict(B=1, H=2, q_len=500, kv_len=500, q_block=128, kv_block=64, mask={"kind": "document"},
         doc_len_min=40, doc_len_max=200),
    dict(B=1, H=3, q_len=400, kv_len=400, q_block=64, kv_block=64,
         score={"kind": "rel_bias", "bias_max": 8.0}, doc_len_min=1, doc_len_max=150),
    # value head dim other than the query / key head dim
    dict(B=1, H=2, q_len=600, kv_len=600, d=64, dv=128, doc_len_min=1, doc_len_max=200),
    dict(B=1, H=2, q_len=450, kv_len=450, d=128, dv=64, q_block=128, kv_block=128,
         doc_len_min=30, doc_len_max=300),
])
def test_backward_parity(over):
    from test_bwd_gpu import check, oracle_bwd
    cfg = workload("document_causal", **over)
    mask = with_doc_ids(cfg)
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    args = (_dev(mask), cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"], out_dtype=torch.bfloat16,
                      return_lse=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg.get("score"), cfg["scale"],
                        dlse=dlse.to(DEV))
    torch.cuda.synchronize()
    got = tuple(t.double().cpu().numpy() for t in (dq, dk, dv))
    cfg2 = dict(cfg, mask=mask)
    ref = oracle_bwd(cfg2, q, k, v, dout, dlse)
    check(got, ref, torch.float32, "document bwd %s" % over)


UNSORTED_CASES = [
    # (q ids, kv ids): a step down in the query ids, in the key ids, and one
    # across the check kernel's 256-thread boundary (positions 255 -> 256)
    (np.r_[[0] * 100, [2] * 60, [1] * 40, [3] * 100], None),
    (np.r_[[0] * 150, [1] * 150], np.r_[[0] * 120, [1] * 60, [0] * 120]),
    (np.r_[[0] * 256, [1] * 344], np.r_[[0] * 100, [1] * 156, [0] * 344]),
]


@pytest.mark.parametrize("qids,kvids", UNSORTED_CASES, ids=["q-step", "kv-step", "kv-boundary"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_unsorted_ids_give_nan(qids, kvids, dtype):
    """Ids that are not non-decreasing break the builder's precondition: it
    lists no tile, every bounds pair is (INT32_MAX, INT32_MIN), and the
    forward and backward write NaN everywhere instead of plausible numbers."""
    q_doc = torch.from_numpy(np.asarray(qids, np.int32))
    kv_doc = q_doc if kvids is None else torch.from_numpy(np.asarray(kvids, np.int32))
    L = int(q_doc.numel())
    assert kv_doc.numel() == L
    cfg = workload("document_causal", B=1, H=2, q_len=L, kv_len=L, q_block=64, kv_block=64,
                   dtype="bf16" if dtype == torch.bfloat16 else "fp32")
    for kind in ("document", "document_causal"):
        print("case", kind, dtype, L, flush=True)
        mask = _dev(_mask(kind, q_doc, kv_doc))
        bm = fa.build_block_mask(mask, L, L, 64, 64, device=DEV)
        bmt = fa.build_block_mask_t(mask, L, L, 64, 64, device=DEV)
        torch.cuda.synchronize()
        for arr in (bm.kv_num_blocks, bm.full_kv_num_blocks, bmt.q_num_blocks, bmt.full_q_num_blocks):
            assert int(arr.abs().sum()) == 0
        for b in (bm.row_bounds, bmt.col_bounds):
            b = b.cpu().view(-1, 2)
            assert bool((b[:, 0] == 2**31 - 1).all()) and bool((b[:, 1] == -2**31).all())
        q, k, v = make_inputs(cfg)
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        for out_dtype in (torch.float32, torch.bfloat16):
            out, lse = fa.fwd(qd, kd, vd, bm, None, cfg["scale"], out_dtype=out_dtype,
                              return_lse=True)
            torch.cuda.synchronize()
            assert bool(out.float().isnan().all()) and bool(lse.isnan().all())
        # the backward takes an output of the inputs' dtype
        out, lse = fa.fwd(qd, kd, vd, bm, None, cfg["scale"], out_dtype=dtype, return_lse=True)
        dout, dlse = make_grad_inputs(cfg, with_dlse=True)
        dq, dk, dv = fa.bwd(qd, kd, vd, out, dout.to(DEV), lse, bm, bmt, None, cfg["scale"],
                            dlse=dlse.to(DEV))
        torch.cuda.synchronize()
        for g in (dq, dk, dv):
            assert bool(g.float().isnan().all())
