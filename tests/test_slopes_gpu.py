"""REL_BIAS with a per-head slope table: a score_mod that closes over a
tensor (the op's score_mod_other_buffers slot in the subtiling page's test
hunks), slope_h = slopes[h] read by the kernels.  Forward (bf16 and fp32
inputs, head dims 64 and 128, both output dtypes) and backward against the
fp64 oracle under the usual bars, and the table holding exactly the
formula's values gives the formula's bits."""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_grad_inputs, make_inputs, workload
from parity import compare, oracle_rows, run_gpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _table(H, seed):
    """Slopes of both signs, a zero, and magnitudes from 2^-9 to 1.5."""
    g = np.random.default_rng(seed)
    t = g.uniform(-0.3, 1.5, H).astype(np.float32)
    t[0] = 0.0
    if H > 2:
        t[2] = 2.0 ** -9
    return torch.from_numpy(t)


FWD = [
    ("causal_rel_bias", dict(B=1, H=4, q_len=700, kv_len=700)),
    ("causal_rel_bias", dict(B=2, H=3, q_len=333, kv_len=333, q_block=128, kv_block=64)),
    ("long_causal_d128", dict(B=1, H=3, q_len=500, kv_len=500)),
    ("prefix_causal", dict(B=1, H=4, q_len=640, kv_len=640, mask={"kind": "sliding_window",
                                                                   "window": 200, "window_min": 0})),
    ("causal_rel_bias", dict(B=1, H=3, q_len=300, kv_len=300, dtype="fp32", q_block=64, kv_block=64)),
]


@pytest.mark.parametrize("name,over", FWD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(FWD)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_forward_with_slope_table(name, over, out_dtype):
    cfg = workload(name, **over)
    if "d" in over or name == "long_causal_d128":
        cfg["scale"] = fa.default_scale(cfg["d"])
    table = _table(cfg["H"], 5)
    cfg["score"] = {"kind": "rel_bias", "slopes": table}
    q, k, v = make_inputs(cfg)
    print("case", name, over, out_dtype, flush=True)
    gcfg = dict(cfg, score={"kind": "rel_bias", "slopes": table.to(DEV)})
    od = {"bf16": torch.bfloat16, "fp32": torch.float32}[out_dtype]
    out, lse, _ = run_gpu(gcfg, q, k, v, out_dtype=od, lse=True)
    ref_out, ref_lse = oracle_rows(cfg, q, k, v)
    D = out.shape[-1]
    compare(out.reshape(-1, D), lse.reshape(-1), ref_out, ref_lse, cfg["dtype"], out_dtype,
            what=name + " slope table")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_table_of_formula_values_gives_the_formula_bits(dtype):
    """With 8 heads and bias_max 8 the formula's slopes are 2^-1 .. 2^-8,
    exact in fp32 on both paths."""
    cfg = workload("causal_rel_bias", B=1, H=8, q_len=520, kv_len=520, dtype=dtype,
                   q_block=64, kv_block=64)
    q, k, v = make_inputs(cfg)
    a = run_gpu(dict(cfg, score={"kind": "rel_bias", "bias_max": 8.0}), q, k, v,
                out_dtype=torch.float32, lse=True)
    table = torch.tensor([2.0 ** -(h + 1) for h in range(8)], dtype=torch.float32, device=DEV)
    b = run_gpu(dict(cfg, score={"kind": "rel_bias", "slopes": table}), q, k, v,
                out_dtype=torch.float32, lse=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


BWD = [
    dict(B=1, H=4, q_len=600, kv_len=600),
    dict(B=1, H=3, q_len=450, kv_len=450, d=128, q_block=128, kv_block=128),
    dict(B=1, H=2, q_len=300, kv_len=300, q_block=64, kv_block=64, d=64, dv=128),
]


@pytest.mark.parametrize("over", BWD)
def test_backward_with_slope_table(over):
    from test_bwd_gpu import check, oracle_bwd
    cfg = workload("causal_rel_bias", **over)
    cfg["scale"] = fa.default_scale(cfg["d"])
    table = _table(cfg["H"], 9)
    cfg["score"] = {"kind": "rel_bias", "slopes": table}
    q, k, v = make_inputs(cfg)
    dout, dlse = make_grad_inputs(cfg, with_dlse=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    print("case", over, flush=True)
    gscore = {"kind": "rel_bias", "slopes": table.to(DEV)}
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(qd, kd, vd, bm, gscore, cfg["scale"], out_dtype=torch.bfloat16,
                      return_lse=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, gscore, cfg["scale"],
                        dlse=dlse.to(DEV))
    torch.cuda.synchronize()
    got = tuple(t.double().cpu().numpy() for t in (dq, dk, dv))
    ref = oracle_bwd(cfg, q, k, v, dout, dlse)
    check(got, ref, torch.float32, "slope table bwd %s" % over)


def test_binding_checks_the_table():
    cfg = workload("causal_rel_bias", B=1, H=4, q_len=128, kv_len=128)
    q, k, v = (t.to(DEV) for t in make_inputs(cfg))
    bm = fa.build_block_mask(cfg["mask"], 128, 128, cfg["q_block"], cfg["kv_block"], device=DEV)
    for bad in (torch.ones(4), torch.ones(3, device=DEV), torch.ones(4, dtype=torch.float64, device=DEV)):
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, bm, {"kind": "rel_bias", "slopes": bad}, cfg["scale"])
