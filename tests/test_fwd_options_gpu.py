"""GPU forward kernel options vs the fp64 oracle, through the C ABI.

The options are the kernel_options entries of the flex_attention op in the
test hunks of "[Inductor][Flex Attention] Add Subtiling Option for Alpha
Scaling"; the page names them without defining them, and the readings tested
here are:

* OUTPUT_MAX: a third output, each row's largest visible score (scaled,
  after the score modification; -inf for a row with no key).  Bar: within
  1e-3 of the oracle's row max (the score comes out of one fp32 dot product
  of exact inputs and a multiply by ln 2; like lse), -inf exactly where the
  oracle has -inf; out and lse of the same call meet the forward's usual bars.
* PRESCALE_QK: q is multiplied by scale * log2 e in fp32 and rounded to the
  input type before Q K^T.  Bar: the usual forward bars against the oracle run
  on those rounded q values with scale ln 2 (the same scores in exact
  arithmetic); and against the plain definition, lse within
  1e-3 + 2^-9 * max_j |scale| sum_d |q_d k_jd| (what rounding q to bf16 can
  move a score by).
* ROWS_GUARANTEED_SAFE, BLOCKS_ARE_CONTIGUOUS: promises by the caller; where
  they hold, results are bitwise identical to the call without them.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_inputs, workload
from oracle import oracle
from parity import compare

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LOG2E = 1.4426950408889634
TOL_MAX = 1e-3


def _run(cfg, q, k, v, **kw):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    bm = fa.build_block_mask(cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"],
                             cfg["kv_block"], device=DEV)
    res = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"], out_dtype=torch.float32,
                 return_lse=True, **kw)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.double().cpu().numpy() for t in res)


def _oracle(cfg, q, k, v, scale=None):
    f = lambda t: t.float().numpy()
    return oracle.attention_rows(f(q), f(k), f(v), cfg["mask"], cfg.get("score", {"kind": "identity"}),
                                 cfg["scale"] if scale is None else scale, with_max=True)


MAX_CASES = [
    ("tiny_causal", {}),
    ("tiny_causal", dict(H=2, q_len=200, kv_len=300, mask={"kind": "noop"})),
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000, mask={"kind": "prefix_causal", "prefix": 300})),
    ("sliding_window", dict(B=1, H=2, q_len=700, kv_len=700, q_block=64, kv_block=64,
                            mask={"kind": "sliding_window", "window": 100, "window_min": 3})),
    ("long_causal_d128", dict(B=1, H=2, q_len=333, kv_len=333)),
    ("causal_rel_bias", dict(B=1, H=8, q_len=700, kv_len=700)),
    ("causal_rel_bias", dict(B=1, H=3, q_len=300, kv_len=300, q_block=128, kv_block=64,
                             mask={"kind": "prefix_causal", "prefix": 100})),
]


@pytest.mark.parametrize("name,over", MAX_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(MAX_CASES)])
def test_output_max(name, over):
    cfg = workload(name, **over)
    cfg["scale"] = fa.default_scale(cfg["d"])
    q, k, v = make_inputs(cfg)
    print("case", name, over, flush=True)
    out, lse, mx = _run(cfg, q, k, v, return_max=True)
    ref_out, ref_lse, ref_mx = _oracle(cfg, q, k, v)
    D = cfg["d"]
    compare(out.reshape(-1, D), lse.reshape(-1), ref_out, ref_lse, cfg["dtype"], "fp32",
            what=name + " (max requested)")
    mx = mx.reshape(-1)
    dead = np.isneginf(ref_mx)
    assert np.array_equal(np.isneginf(mx), dead), "rows with no key differ"
    err = float(np.abs(mx[~dead] - ref_mx[~dead]).max()) if (~dead).any() else 0.0
    print("  max err %.2e" % err, flush=True)
    assert err <= TOL_MAX
    # max <= lse on every live row (up to the two tolerances)
    assert np.all(mx[~dead] <= lse.reshape(-1)[~dead] + TOL_MAX + 1e-3)


def test_output_max_negative_scale_and_subtiling():
    cfg = workload("prefix_causal", B=1, H=2, q_len=400, kv_len=400, q_block=128, kv_block=128)
    cfg["scale"] = -0.2
    q, k, v = make_inputs(cfg)
    out, lse, mx = _run(cfg, q, k, v, return_max=True)
    out_s, lse_s, mx_s = _run(cfg, q, k, v, return_max=True, use_subtiling=True)
    # subtiling only reorders the rescale: bitwise the same
    assert np.array_equal(out, out_s) and np.array_equal(lse, lse_s) and np.array_equal(mx, mx_s)
    ref_out, ref_lse, ref_mx = _oracle(cfg, q, k, v)
    compare(out.reshape(-1, 64), lse.reshape(-1), ref_out, ref_lse, "bf16", "fp32", what="neg max")
    assert np.abs(mx.reshape(-1) - ref_mx).max() <= TOL_MAX


def test_output_max_full_size_sampled():
    """The sliding-window workload at full size with the max requested; the
    oracle checks sampled rows."""
    from parity import sample_rows
    cfg = workload("sliding_window")
    q, k, v = make_inputs(cfg)
    out, lse, mx = _run(cfg, q, k, v, return_max=True)
    rows = sample_rows(cfg)
    f = lambda t: t.float().numpy()
    ref_out, ref_lse, ref_mx = oracle.attention_rows(f(q), f(k), f(v), cfg["mask"], cfg["score"],
                                                     cfg["scale"], rows=rows, with_max=True)
    compare(out.reshape(-1, 64)[rows], lse.reshape(-1)[rows], ref_out, ref_lse, "bf16", "fp32",
            what="full sliding max")
    assert np.abs(mx.reshape(-1)[rows] - ref_mx).max() <= TOL_MAX


def _prescaled_q(q, scale):
    """q * (scale * log2 e) in fp32, rounded back to q's dtype (RNE)."""
    f = np.float32(float(np.float32(scale)) * LOG2E)
    return (q.float() * torch.tensor(f, dtype=torch.float32)).to(q.dtype)


PRESCALE_CASES = [
    ("tiny_causal", {}),  # fp32 inputs
    ("prefix_causal", dict(B=1, H=2, q_len=520, kv_len=520, mask={"kind": "prefix_causal", "prefix": 256})),
    ("sliding_window", dict(B=1, H=2, q_len=700, kv_len=700)),
    ("long_causal_d128", dict(B=1, H=2, q_len=300, kv_len=300)),
    ("causal_rel_bias", dict(B=1, H=8, q_len=500, kv_len=500)),
]


@pytest.mark.parametrize("name,over", PRESCALE_CASES,
                         ids=[f"{n}-{i}" for i, (n, _) in enumerate(PRESCALE_CASES)])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_prescale_qk(name, over, sign):
    cfg = workload(name, **over)
    cfg["scale"] = sign * fa.default_scale(cfg["d"])
    q, k, v = make_inputs(cfg)
    print("case", name, over, sign, flush=True)
    out, lse = _run(cfg, q, k, v, prescale_qk=True)
    D = cfg["d"]
    # (a) the same scores in exact arithmetic: rounded prescaled q, scale ln 2
    q2 = _prescaled_q(q, cfg["scale"])
    ref_out, ref_lse, _ = _oracle(cfg, q2, k, v, scale=math.log(2.0))
    compare(out.reshape(-1, D), lse.reshape(-1), ref_out, ref_lse, cfg["dtype"], "fp32",
            what=name + " prescaled")
    # (b) against the plain definition, with what rounding q can move a score by
    ref_out0, ref_lse0, _ = _oracle(cfg, q, k, v)
    qa, ka = np.abs(q.double().numpy()), np.abs(k.double().numpy())
    bound = abs(cfg["scale"]) * np.einsum("bhid,bhjd->bhij", qa, ka).max(axis=-1).reshape(-1)
    rnd = 2.0 ** -9 if cfg["dtype"] == "bf16" else 2.0 ** -24
    live = ~np.isneginf(ref_lse0)
    excess = np.abs(lse.reshape(-1) - ref_lse0)[live] - (1e-3 + rnd * bound[live])
    assert excess.max() <= 0.0


@pytest.mark.parametrize("name,over", [
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000, mask={"kind": "prefix_causal", "prefix": 300})),
    ("causal_rel_bias", dict(B=1, H=4, q_len=600, kv_len=600)),
    ("tiny_causal", {}),
])
def test_rows_guaranteed_safe_is_bitwise_neutral(name, over):
    """Every row of a causal or prefix mask sees at least its own key."""
    cfg = workload(name, **over)
    q, k, v = make_inputs(cfg)
    a = _run(cfg, q, k, v)
    b = _run(cfg, q, k, v, rows_guaranteed_safe=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name,over", [
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000, mask={"kind": "causal"})),
    ("prefix_causal", dict(B=1, H=1, q_len=300, kv_len=650, mask={"kind": "noop"})),
    ("causal_rel_bias", dict(B=1, H=2, q_len=777, kv_len=777, q_block=128, kv_block=64)),
    ("tiny_causal", {}),
])
def test_blocks_are_contiguous_is_bitwise_neutral(name, over):
    """Causal and no-mask lists are runs of consecutive kv-blocks (checked on
    the host first); reading only each list's first entry changes nothing."""
    cfg = workload(name, **over)
    bm = fa.build_block_mask(cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"],
                             cfg["kv_block"], device=DEV)
    torch.cuda.synchronize()
    num, idx, fnum, fidx = (t.cpu().numpy() for t in bm.arrays())
    for qb in range(num.shape[0]):
        for n_, ix in ((num[qb], idx[qb]), (fnum[qb], fidx[qb])):
            assert np.array_equal(ix[:n_], ix[0] + np.arange(n_)), "precondition: contiguous lists"
    q, k, v = make_inputs(cfg)
    a = _run(cfg, q, k, v)
    b = _run(cfg, q, k, v, blocks_are_contiguous=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
