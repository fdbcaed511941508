"""GPU backward (dq, dk, dv) vs the fp64 oracle, through the C ABI.

The HIP backward takes the forward's bf16 output and float32 lse as they come
out of the HIP forward, and rounds p and ds to bf16 before the products with
dout^T, q^T and K^T (fp32 accumulation).  Each of those roundings moves one
term of a gradient sum by at most 2^-9 of itself, lse (within 1e-3) moves
every p of a row by the same factor of at most 1e-3, and the bf16 output moves
delta by about 2^-9 sqrt(D) |dout| |out|, small beside dP.  So the error of
each gradient tensor is a small fraction of that tensor's size, and the bar,
per tensor, is

    max |g - ref| <= 1e-2 * max |ref|          (fp32 gradients)

plus half a bf16 ulp of ref for bf16 gradients (the store rounds once more),
plus 1e-5 absolute: where a tensor vanishes because its terms cancel exactly
(a row that sees a single key has ds = dP - delta = 0), the fp32 difference
still leaves about 2^-23 |dP| per term (|dP| <~ 10, times |scale k| <~ 1).
Rows that see no key get dq exactly 0 and keys no query sees get dk = dv = 0
(checked where the mask makes them so; a gradient that is 0 only because its
terms cancel is held to the bar above like any other).
"""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_grad_inputs, make_inputs, workload
from oracle import oracle
from parity import bf16_half_ulp

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-2
ATOL_BWD = 1e-5
DEV = torch.device("cuda:0")


def run_bwd(cfg, q, k, v, dout, dlse=None, grad_dtype=torch.float32, scale=None):
    """HIP forward (bf16 out, lse) then HIP backward.  Returns dq, dk, dv as
    float64 numpy arrays."""
    scale = cfg["scale"] if scale is None else scale
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    dld = dlse.to(DEV) if dlse is not None else None
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg.get("score"), scale, out_dtype=torch.bfloat16,
                      return_lse=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg.get("score"), scale,
                        dlse=dld, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in (dq, dk, dv))


def oracle_bwd(cfg, q, k, v, dout, dlse=None, scale=None, heads=None):
    f = lambda t: t.float().numpy()
    return oracle.attention_backward(
        f(q), f(k), f(v), f(dout), cfg["mask"], cfg.get("score", {"kind": "identity"}),
        cfg["scale"] if scale is None else scale,
        dlse=dlse.numpy() if dlse is not None else None, heads=heads)


def check(got, ref, grad_dtype, what, heads=None):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        if heads is not None:
            B, H = g.shape[:2]
            g = g.reshape(B * H, *g.shape[2:])[heads]
            r = r.reshape(B * H, *r.shape[2:])[heads]
        assert g.shape == r.shape, (name, g.shape, r.shape)
        if g.size == 0:
            errs.append(0.0)
            continue
        assert np.all(np.isfinite(g)), "%s %s: non-finite gradient" % (what, name)
        scale_ref = float(np.abs(r).max())
        err = np.abs(g - r)
        bound = TOL_BWD * scale_ref + ATOL_BWD
        if grad_dtype == torch.bfloat16:
            bound = bound + bf16_half_ulp(r)
        worst = float((err - bound).max())
        rel = float(err.max()) / scale_ref if scale_ref > 0 else float(err.max())
        assert worst <= 0.0, "%s %s: err %.3g of max|ref| %.3g (bar %g)" % (
            what, name, rel, scale_ref, TOL_BWD)
        errs.append(rel)
    print("  %s: max err / max|ref| dq %.2e dk %.2e dv %.2e" % (what, *errs), flush=True)
    return errs


def _case(name, over, grad_dtype=torch.float32, with_dlse=False, scale=None):
    cfg = workload(name, **over)
    cfg["dtype"] = "bf16"
    cfg["scale"] = fa.default_scale(cfg["d"]) if scale is None else scale
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=with_dlse)
    print("case", name, over, grad_dtype, "dlse" if with_dlse else "", flush=True)
    got = run_bwd(cfg, q, k, v, dout, dlse, grad_dtype)
    ref = oracle_bwd(cfg, q, k, v, dout, dlse)
    return check(got, ref, grad_dtype, "%s %s" % (name, over))


# several tiles in both directions and ragged tails; every block pair
SMALL = [
    ("tiny_causal", dict(H=2, q_len=256, kv_len=256)),
    ("tiny_causal", dict(q_len=200, kv_len=200, q_block=128, kv_block=128)),
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000, mask={"kind": "prefix_causal", "prefix": 300})),
    ("prefix_causal", dict(B=2, H=1, q_len=520, kv_len=520, q_block=128, kv_block=128,
                           mask={"kind": "prefix_causal", "prefix": 256})),
    ("prefix_causal", dict(B=1, H=1, q_len=333, kv_len=333, q_block=64, kv_block=64,
                           mask={"kind": "prefix_causal", "prefix": 0})),
    ("sliding_window", dict(B=1, H=2, q_len=1100, kv_len=1100)),
    ("sliding_window", dict(B=1, H=1, q_len=700, kv_len=700, q_block=64, kv_block=64,
                            mask={"kind": "sliding_window", "window": 100, "window_min": 3})),
    ("sliding_window", dict(B=1, H=1, q_len=600, kv_len=600, q_block=128, kv_block=64,
                            mask={"kind": "sliding_window", "window": 40, "window_min": 40})),
    ("causal_rel_bias", dict(B=1, H=8, q_len=700, kv_len=700)),
    ("causal_rel_bias", dict(B=1, H=3, q_len=333, kv_len=333, q_block=128, kv_block=64)),
    ("prefix_causal", dict(B=1, H=2, q_len=300, kv_len=650, mask={"kind": "noop"})),
    ("prefix_causal", dict(B=1, H=1, q_len=650, kv_len=300, mask={"kind": "causal"},
                           q_block=64, kv_block=64)),
    ("prefix_causal", dict(B=1, H=1, q_len=300, kv_len=650, mask={"kind": "causal"},
                           q_block=128, kv_block=128)),
    ("tiny_causal", dict(q_len=1, kv_len=1)),
    ("tiny_causal", dict(q_len=33, kv_len=97, mask={"kind": "noop"})),
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
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_small_parity(name, over):
    _case(name, over)


@pytest.mark.parametrize("i", [0, 2, 6, 8, 15, 17])
def test_small_parity_bf16_grads(i):
    name, over = SMALL[i]
    _case(name, over, grad_dtype=torch.bfloat16)


@pytest.mark.parametrize("i", [3, 6, 9, 16, 18])
def test_lse_gradient(i):
    name, over = SMALL[i]
    _case(name, over, with_dlse=True)


def test_negative_scale():
    _case("prefix_causal", dict(B=1, H=1, q_len=300, kv_len=300), scale=-0.2)
    _case("causal_rel_bias", dict(B=1, H=2, q_len=200, kv_len=200), scale=-0.1)


def test_empty_key_range():
    """kv_len = 0: every row sees no key (out 0, lse -inf); dq is 0."""
    B, H, Lq, D = 1, 2, 70, 64
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    q, out = torch.randn(B, H, Lq, D, device=DEV).bfloat16(), z(B, H, Lq, D)
    dout = torch.randn(B, H, Lq, D, device=DEV).bfloat16()
    k = v = z(B, H, 0, D)
    lse = torch.full((B, H, Lq), float("-inf"), device=DEV)
    bm = fa.build_block_mask({"kind": "causal"}, Lq, 0, 64, 64, device=DEV)
    bmt = fa.build_block_mask_t({"kind": "causal"}, Lq, 0, 64, 64, device=DEV)
    dq, dk, dv = fa.bwd(q, k, v, out, dout, lse, bm, bmt)
    torch.cuda.synchronize()
    assert dk.numel() == 0 and dv.numel() == 0
    assert torch.all(dq == 0)


def test_empty_query_range():
    """q_len = 0: no query sees any key; dk and dv are 0."""
    B, H, Lk, D = 2, 1, 150, 64
    k = torch.randn(B, H, Lk, D, device=DEV).bfloat16()
    v = torch.randn(B, H, Lk, D, device=DEV).bfloat16()
    e = torch.zeros(B, H, 0, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(B, H, 0, device=DEV)
    bm = fa.build_block_mask({"kind": "noop"}, 0, Lk, 128, 64, device=DEV)
    bmt = fa.build_block_mask_t({"kind": "noop"}, 0, Lk, 128, 64, device=DEV)
    dk = torch.full((B, H, Lk, D), 7.0, device=DEV)
    dv = torch.full((B, H, Lk, D), 7.0, device=DEV)
    fa.bwd(e, k, v, e, e, lse, bm, bmt, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_fully_masked_rows_and_keys():
    """window_min = 5 hides every key from rows 0..4 and the last five keys
    from every row: those dq rows and dk / dv rows are exactly 0."""
    cfg = workload("sliding_window", B=1, H=1, q_len=300, kv_len=300, q_block=64, kv_block=64,
                   mask={"kind": "sliding_window", "window": 60, "window_min": 5})
    q, k, v = make_inputs(cfg)
    dout, _ = make_grad_inputs(cfg)
    dq, dk, dv = run_bwd(cfg, q, k, v, dout)
    assert np.all(dq[:, :, :5] == 0.0)
    assert np.all(dk[:, :, -5:] == 0.0) and np.all(dv[:, :, -5:] == 0.0)
    ref = oracle_bwd(cfg, q, k, v, dout)
    check((dq, dk, dv), ref, torch.float32, "fully masked")


# value head dim Dv other than the query / key head dim D (v, out, dout and
# dv are Dv wide): both orders, every tile shape, ragged tails
DV_CASES = [
    ("prefix_causal", dict(B=1, H=2, q_len=777, kv_len=777, d=64, dv=128,
                           mask={"kind": "prefix_causal", "prefix": 300})),
    ("prefix_causal", dict(B=1, H=1, q_len=333, kv_len=333, d=64, dv=128, q_block=64, kv_block=64,
                           mask={"kind": "causal"})),
    ("prefix_causal", dict(B=1, H=1, q_len=520, kv_len=520, d=64, dv=128, q_block=128,
                           kv_block=128, mask={"kind": "sliding_window", "window": 150,
                                               "window_min": 2})),
    ("prefix_causal", dict(B=1, H=2, q_len=600, kv_len=600, d=128, dv=64,
                           mask={"kind": "causal"})),
    ("prefix_causal", dict(B=1, H=1, q_len=300, kv_len=650, d=128, dv=64, q_block=64,
                           kv_block=64, mask={"kind": "noop"})),
    ("prefix_causal", dict(B=1, H=1, q_len=450, kv_len=450, d=128, dv=64, q_block=128,
                           kv_block=128, mask={"kind": "prefix_causal", "prefix": 100})),
    ("causal_rel_bias", dict(B=1, H=4, q_len=260, kv_len=260, d=64, dv=128)),
    ("causal_rel_bias", dict(B=1, H=4, q_len=260, kv_len=260, d=128, dv=64, q_block=128,
                             kv_block=64)),
]


@pytest.mark.parametrize("name,over", DV_CASES,
                         ids=[f"{n}-{o['d']}-{o['dv']}-{i}" for i, (n, o) in enumerate(DV_CASES)])
def test_value_head_dim_parity(name, over):
    _case(name, over)


@pytest.mark.parametrize("i", [0, 3])
def test_value_head_dim_bf16_grads_and_lse_gradient(i):
    name, over = DV_CASES[i]
    _case(name, over, grad_dtype=torch.bfloat16, with_dlse=True)


# ---- full-size workloads in the benchmark's launch configuration; the oracle
# computes the first and last head (heads are independent) ----


@pytest.mark.parametrize("name", ["prefix_causal", "sliding_window"])
def test_full_size_sampled_heads(name):
    cfg = workload(name)
    q, k, v = make_inputs(cfg)
    dout, _ = make_grad_inputs(cfg)
    print("case full", name, flush=True)
    got = run_bwd(cfg, q, k, v, dout)
    nh = cfg["B"] * cfg["H"]
    heads = [0, nh - 1]
    # the oracle only on those heads' slices
    ref = oracle_bwd(cfg, q, k, v, dout, heads=heads)
    check(got, ref, torch.float32, "full " + name, heads=heads)


def test_long_causal_d128_4k_sampled_heads():
    """The head-dim-128 workload's settings at 4096 tokens, first and last head."""
    cfg = workload("long_causal_d128", q_len=4096, kv_len=4096)
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=True)
    print("case d128 4k", flush=True)
    got = run_bwd(cfg, q, k, v, dout, dlse)
    heads = [0, cfg["B"] * cfg["H"] - 1]
    ref = oracle_bwd(cfg, q, k, v, dout, dlse, heads=heads)
    check(got, ref, torch.float32, "d128 4k", heads=heads)


def test_rel_bias_4k():
    """The relative-bias workload's settings at 4096 tokens, all heads."""
    cfg = workload("causal_rel_bias", B=1, q_len=4096, kv_len=4096)
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=True)
    print("case rel_bias 4k", flush=True)
    got = run_bwd(cfg, q, k, v, dout, dlse)
    ref = oracle_bwd(cfg, q, k, v, dout, dlse)
    check(got, ref, torch.float32, "rel_bias 4k")


@pytest.mark.parametrize("name,over", [
    ("prefix_causal", dict(B=2, H=2, q_len=333, kv_len=301, mask={"kind": "prefix_causal", "prefix": 100})),
    ("sliding_window", dict(B=1, H=3, q_len=461, kv_len=461)),
    ("long_causal_d128", dict(B=1, H=2, q_len=297, kv_len=297)),
    ("prefix_causal", dict(B=1, H=2, q_len=201, kv_len=201, dv=128, mask={"kind": "causal"})),
    ("long_causal_d128", dict(B=1, H=1, q_len=150, kv_len=230, dv=64, q_block=128, kv_block=64,
                              mask={"kind": "noop"})),
])
def test_bf16_grads_stay_inside_their_tensors(name, over):
    """bf16 dq, dk, dv of ragged lengths: they match the oracle, and nothing
    past the end of any gradient tensor is written."""
    cfg = workload(name, **over)
    cfg["scale"] = fa.default_scale(cfg["d"])
    q, k, v = make_inputs(cfg)
    dout, _ = make_grad_inputs(cfg)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], out_dtype=torch.bfloat16,
                      return_lse=True)
    pad = 64 * 1024
    sentinel = -12345.0  # exact in bf16
    grads = []
    for shape in (qd.shape, kd.shape, vd.shape):
        n = int(np.prod(shape))
        flat = torch.full((n + pad,), sentinel, dtype=torch.bfloat16, device=DEV)
        grads.append((flat, flat[:n].view(shape)))
    fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg["score"], cfg["scale"],
           grad_dtype=torch.bfloat16, dq=grads[0][1], dk=grads[1][1], dv=grads[2][1])
    torch.cuda.synchronize()
    for nm, (flat, g) in zip(("dq", "dk", "dv"), grads):
        assert bool((flat[g.numel():] == sentinel).all()), "write past the end of " + nm
    got = tuple(g.double().cpu().numpy() for _, g in grads)
    check(got, oracle_bwd(cfg, q, k, v, dout), torch.bfloat16, "%s %s" % (name, over))


@pytest.mark.parametrize("name,over", [
    ("prefix_causal", dict(B=1, H=2, q_len=333, kv_len=333, mask={"kind": "prefix_causal", "prefix": 100})),
    ("long_causal_d128", dict(B=1, H=2, q_len=300, kv_len=300)),
    ("sliding_window", dict(B=1, H=2, q_len=461, kv_len=461, dv=128)),
])
def test_write_dq_off(name, over):
    """WRITE_DQ off (dq = NULL): the launcher skips the dq kernel, and dk
    and dv are bitwise the same as with dq requested (and within the
    backward bar of the oracle)."""
    cfg = workload(name, **over)
    q, k, v = make_inputs(cfg)
    dout, _ = make_grad_inputs(cfg)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"], return_lse=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg.get("score"), cfg["scale"],
                        grad_dtype=torch.bfloat16)
    none, dk2, dv2 = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg.get("score"), cfg["scale"],
                            grad_dtype=torch.bfloat16, write_dq=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # and the gradients themselves are the oracle's (dk, dv)
    refs = oracle_bwd(cfg, q, k, v, dout)
    for name_g, g, r in (("dk", dk2, refs[1]), ("dv", dv2, refs[2])):
        gn = g.double().cpu().numpy()
        bound = TOL_BWD * np.abs(r).max() + ATOL_BWD + bf16_half_ulp(r)
        assert np.all(np.abs(gn - r) <= bound), name_g
