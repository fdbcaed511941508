"""GPU backward for fp32 inputs (dq, dk, dv) vs the fp64 oracle, through the
C ABI.

The fp32 forward's output and lse feed the fp32 backward; every product and
sum is fp32 (no bf16 rounding anywhere).  Each gradient element is a sum of
at most kv_len (q_len) terms, each a product of a p or ds with an input row;
p carries the lse error (the forward's, about 1e-6 of |s|) and one exp
rounding, ds = p (dP - delta) the fp32 errors of two dot products of length
D.  The fp32 sum of n terms is within n 2^-24 of the sum of their sizes, so
beside the tensor's largest entry the error stays a few 1e-6; the bar is the
forward's fp32 one,

    max |g - ref| <= 1e-4 * max |ref| + 1e-5 (absolute, for entries whose
    terms cancel: a row seeing one key has ds = dP - delta = 0 exactly in the
    oracle but about 2^-24 |dP| per term in fp32)

plus half a bf16 ulp of ref for bf16 gradients.  Cases span every mask kind,
both head dims, value head dims unlike them, every tile shape, ragged tails
on both sides, the relative
bias (formula and per-head table), the lse gradient, a negative scale,
WRITE_DQ off, empty ranges and unsorted document ids."""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import (make_grad_inputs, make_inputs,
                                                          with_doc_ids, workload)
from oracle import oracle
from parity import bf16_half_ulp

pytestmark = pytest.mark.gpu

TOL = 1e-4
ATOL = 1e-5
DEV = torch.device("cuda:0")


def _dev_mask(mask):
    if "q_doc" not in mask:
        return mask
    return dict(mask, q_doc=mask["q_doc"].to(DEV), kv_doc=mask["kv_doc"].to(DEV))


def _gpu_score(score):
    if score and "slopes" in score:
        return dict(score, slopes=score["slopes"].to(DEV))
    return score


def run(cfg, mask, q, k, v, dout, dlse=None, grad_dtype=torch.float32, write_dq=True):
    """HIP fp32 forward (fp32 out and lse), then the HIP fp32 backward."""
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    args = (_dev_mask(mask), cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    sc = _gpu_score(cfg.get("score"))
    out, lse = fa.fwd(qd, kd, vd, bm, sc, cfg["scale"], out_dtype=torch.float32, return_lse=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, sc, cfg["scale"],
                        dlse=dlse.to(DEV) if dlse is not None else None, grad_dtype=grad_dtype,
                        write_dq=write_dq)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.double().cpu().numpy() for t in (dq, dk, dv))


def reference(cfg, mask, q, k, v, dout, dlse=None):
    f = lambda t: t.numpy().astype(np.float32)
    return oracle.attention_backward(
        f(q), f(k), f(v), f(dout), mask, cfg.get("score", {"kind": "identity"}), cfg["scale"],
        dlse=dlse.numpy() if dlse is not None else None)


def check(got, ref, grad_dtype, what):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        if g is None:
            errs.append(float("nan"))
            continue
        assert g.shape == r.shape, (name, g.shape, r.shape)
        if g.size == 0:
            errs.append(0.0)
            continue
        assert np.all(np.isfinite(g)), "%s %s: non-finite gradient" % (what, name)
        top = float(np.abs(r).max())
        err = np.abs(g - r)
        bound = TOL * top + ATOL
        if grad_dtype == torch.bfloat16:
            bound = bound + bf16_half_ulp(r)
        rel = float(err.max()) / top if top > 0 else float(err.max())
        assert float((err - bound).max()) <= 0.0, "%s %s: err %.3g of max|ref| %.3g (bar %g)" % (
            what, name, rel, top, TOL)
        errs.append(rel)
    print("  %s: max err / max|ref| dq %.2e dk %.2e dv %.2e" % (what, *errs), flush=True)
    return errs


def _case(name, over, grad_dtype=torch.float32, with_dlse=False, scale=None, write_dq=True):
    cfg = workload(name, **over)
    cfg["dtype"] = "fp32"
    cfg["scale"] = fa.default_scale(cfg["d"]) if scale is None else scale
    mask = with_doc_ids(cfg)
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=with_dlse)
    assert q.dtype == torch.float32 and dout.dtype == torch.float32
    print("case", name, over, grad_dtype, "dlse" if with_dlse else "", scale, write_dq, flush=True)
    got = run(cfg, mask, q, k, v, dout, dlse, grad_dtype, write_dq)
    ref = reference(cfg, mask, q, k, v, dout, dlse)
    return check(got, ref, grad_dtype, "%s %s" % (name, over))


CASES = [
    ("tiny_causal", dict(H=2, q_len=256, kv_len=256)),
    ("tiny_causal", dict(q_len=200, kv_len=200, q_block=128, kv_block=128)),
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000,
                           mask={"kind": "prefix_causal", "prefix": 300})),
    ("prefix_causal", dict(B=2, H=1, q_len=520, kv_len=520, q_block=128, kv_block=128,
                           mask={"kind": "prefix_causal", "prefix": 256})),
    ("sliding_window", dict(B=1, H=1, q_len=700, kv_len=700, q_block=64, kv_block=64,
                            mask={"kind": "sliding_window", "window": 100, "window_min": 3})),
    ("sliding_window", dict(B=1, H=2, q_len=900, kv_len=900, q_block=128, kv_block=64)),
    ("causal_rel_bias", dict(B=1, H=3, q_len=333, kv_len=333, q_block=128, kv_block=64)),
    ("prefix_causal", dict(B=1, H=2, q_len=300, kv_len=650, mask={"kind": "noop"})),
    ("prefix_causal", dict(B=1, H=1, q_len=650, kv_len=300, mask={"kind": "causal"},
                           q_block=64, kv_block=64)),
    ("tiny_causal", dict(q_len=1, kv_len=1)),
    ("tiny_causal", dict(q_len=33, kv_len=97, mask={"kind": "noop"})),
    ("document_causal", dict(B=1, H=2, q_len=700, kv_len=700, doc_len_min=1, doc_len_max=260)),
    ("document_causal", dict(B=1, H=2, q_len=500, kv_len=500, q_block=128, kv_block=64,
                             mask={"kind": "document"}, doc_len_min=40, doc_len_max=200)),
    # head dim 128, every tile shape
    ("long_causal_d128", dict(B=1, H=2, q_len=300, kv_len=300)),
    ("long_causal_d128", dict(B=1, H=2, q_len=520, kv_len=520, q_block=128, kv_block=64,
                              mask={"kind": "prefix_causal", "prefix": 200})),
    ("long_causal_d128", dict(B=1, H=1, q_len=333, kv_len=333, q_block=64, kv_block=64,
                              mask={"kind": "sliding_window", "window": 90, "window_min": 2})),
    ("long_causal_d128", dict(B=1, H=4, q_len=260, kv_len=260,
                              score={"kind": "rel_bias", "bias_max": 8.0})),
    ("long_causal_d128", dict(B=1, H=1, q_len=200, kv_len=450, mask={"kind": "noop"},
                              q_block=128, kv_block=64)),
    # value head dim unlike the key head dim, every tile shape
    ("prefix_causal", dict(B=1, H=2, q_len=520, kv_len=520, dv=128,
                           mask={"kind": "prefix_causal", "prefix": 200})),
    ("sliding_window", dict(B=1, H=1, q_len=700, kv_len=700, dv=128, q_block=128, kv_block=64,
                            mask={"kind": "sliding_window", "window": 100, "window_min": 3})),
    ("document_causal", dict(B=1, H=2, q_len=500, kv_len=500, dv=128, q_block=128, kv_block=128,
                             doc_len_min=1, doc_len_max=200)),
    ("long_causal_d128", dict(B=1, H=2, q_len=333, kv_len=333, dv=64)),
    ("long_causal_d128", dict(B=1, H=3, q_len=300, kv_len=300, dv=64, q_block=128, kv_block=64,
                              score={"kind": "rel_bias", "bias_max": 8.0})),
    ("long_causal_d128", dict(B=1, H=1, q_len=200, kv_len=450, dv=64, mask={"kind": "noop"},
                              q_block=64, kv_block=64)),
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_fp32_parity(name, over):
    _case(name, over)


@pytest.mark.parametrize("i", [0, 4, 13, 19, 21])
def test_fp32_bf16_grads(i):
    name, over = CASES[i]
    _case(name, over, grad_dtype=torch.bfloat16)


@pytest.mark.parametrize("i", [2, 6, 11, 16, 20, 22])
def test_fp32_lse_gradient(i):
    name, over = CASES[i]
    _case(name, over, with_dlse=True)


def test_fp32_negative_scale():
    _case("prefix_causal", dict(B=1, H=1, q_len=300, kv_len=300), scale=-0.2)
    _case("causal_rel_bias", dict(B=1, H=2, q_len=200, kv_len=200), scale=-0.1)


def test_fp32_slope_table():
    table = torch.tensor([0.0, 0.7, 2.0 ** -9, -0.25], dtype=torch.float32)
    _case("causal_rel_bias", dict(B=1, H=4, q_len=300, kv_len=300,
                                  score={"kind": "rel_bias", "slopes": table}))


@pytest.mark.parametrize("i", [3, 14, 23])
def test_fp32_write_dq_off(i):
    """WRITE_DQ off: no dq, and dk / dv bit-identical to the run with dq."""
    name, over = CASES[i]
    cfg = workload(name, **over)
    cfg["dtype"] = "fp32"
    cfg["scale"] = fa.default_scale(cfg["d"])
    mask = with_doc_ids(cfg)
    q, k, v = make_inputs(cfg)
    dout, _ = make_grad_inputs(cfg)
    print("case", name, over, flush=True)
    full = run(cfg, mask, q, k, v, dout)
    part = run(cfg, mask, q, k, v, dout, write_dq=False)
    assert part[0] is None
    assert np.array_equal(full[1], part[1]) and np.array_equal(full[2], part[2])


def test_fp32_empty_ranges():
    """kv_len = 0: dq is 0; q_len = 0: dk and dv are 0."""
    B, H, D = 1, 2, 64
    q = torch.randn(B, H, 70, D, device=DEV)
    dout = torch.randn(B, H, 70, D, device=DEV)
    out = torch.zeros(B, H, 70, D, device=DEV)
    e = torch.zeros(B, H, 0, D, device=DEV)
    lse = torch.full((B, H, 70), float("-inf"), device=DEV)
    bm = fa.build_block_mask({"kind": "causal"}, 70, 0, 64, 64, device=DEV)
    bmt = fa.build_block_mask_t({"kind": "causal"}, 70, 0, 64, 64, device=DEV)
    dq, dk, dv = fa.bwd(q, e, e, out, dout, lse, bm, bmt)
    torch.cuda.synchronize()
    assert dk.numel() == 0 and dv.numel() == 0 and bool(torch.all(dq == 0))
    k = torch.randn(B, H, 150, D, device=DEV)
    v = torch.randn(B, H, 150, D, device=DEV)
    bm = fa.build_block_mask({"kind": "noop"}, 0, 150, 128, 64, device=DEV)
    bmt = fa.build_block_mask_t({"kind": "noop"}, 0, 150, 128, 64, device=DEV)
    dk = torch.full((B, H, 150, D), 7.0, device=DEV)
    dv = torch.full((B, H, 150, D), 7.0, device=DEV)
    fa.bwd(e, k, v, e, e, torch.zeros(B, H, 0, device=DEV), bm, bmt, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert bool(torch.all(dk == 0)) and bool(torch.all(dv == 0))


def test_fp32_empty_ranges_value_head_dim():
    """As above with value head dims unlike the key's.  kv_len = 0 with
    D = 128, Dv = 64: the forward writes out 0 and lse -inf, dq is 0;
    q_len = 0 with D = 64, Dv = 128: dk (64 wide) and dv (128 wide) are 0."""
    B, H = 1, 2
    q = torch.randn(B, H, 70, 128, device=DEV)
    ek, ev = torch.zeros(B, H, 0, 128, device=DEV), torch.zeros(B, H, 0, 64, device=DEV)
    bm = fa.build_block_mask({"kind": "causal"}, 70, 0, 64, 64, device=DEV)
    bmt = fa.build_block_mask_t({"kind": "causal"}, 70, 0, 64, 64, device=DEV)
    out = torch.full((B, H, 70, 64), 7.0, device=DEV)
    lse = torch.zeros(B, H, 70, device=DEV)
    fa.fwd(q, ek, ev, bm, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0)) and bool(torch.all(torch.isneginf(lse)))
    dout = torch.randn(B, H, 70, 64, device=DEV)
    dq, dk, dv = fa.bwd(q, ek, ev, out, dout, lse, bm, bmt)
    torch.cuda.synchronize()
    assert dk.numel() == 0 and dv.numel() == 0 and dq.shape == q.shape
    assert bool(torch.all(dq == 0))
    k = torch.randn(B, H, 150, 64, device=DEV)
    v = torch.randn(B, H, 150, 128, device=DEV)
    eq, eo = torch.zeros(B, H, 0, 64, device=DEV), torch.zeros(B, H, 0, 128, device=DEV)
    bm = fa.build_block_mask({"kind": "noop"}, 0, 150, 128, 128, device=DEV)
    bmt = fa.build_block_mask_t({"kind": "noop"}, 0, 150, 128, 128, device=DEV)
    dk = torch.full((B, H, 150, 64), 7.0, device=DEV)
    dv = torch.full((B, H, 150, 128), 7.0, device=DEV)
    fa.bwd(eq, k, v, eo, eo, torch.zeros(B, H, 0, device=DEV), bm, bmt, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert bool(torch.all(dk == 0)) and bool(torch.all(dv == 0))


def test_fp32_fully_masked_rows_and_keys():
    """window_min = 5 hides every key from rows 0..4 and the last five keys
    from every row: those dq rows and dk / dv rows are exactly 0."""
    cfg = workload("sliding_window", B=1, H=1, q_len=300, kv_len=300, q_block=64, kv_block=64,
                   mask={"kind": "sliding_window", "window": 60, "window_min": 5})
    cfg["dtype"] = "fp32"
    q, k, v = make_inputs(cfg)
    dout, _ = make_grad_inputs(cfg)
    dq, dk, dv = run(cfg, cfg["mask"], q, k, v, dout)
    assert np.all(dq[:, :, :5] == 0.0)
    assert np.all(dk[:, :, -5:] == 0.0) and np.all(dv[:, :, -5:] == 0.0)


@pytest.mark.parametrize("seed", range(500, 516))
def test_fp32_random_case(seed):
    """Seeded random draws (mask kind and parameters, score modification, head
    dims, tile shape, ragged and unequal lengths, gradient dtype, lse
    gradient) as in the bf16 sweep, with fp32 inputs."""
    from test_bwd_random_gpu import _case as draw
    over, grad_dtype, with_dlse = draw(seed)
    _case("prefix_causal", over, grad_dtype=grad_dtype, with_dlse=with_dlse)
