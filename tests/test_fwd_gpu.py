"""GPU forward vs the fp64 oracle, through the C ABI.

Tolerances (see tests/parity.py): bf16 inputs -> out max-abs 1e-2 (fp32 out;
bf16 out adds half a bf16 ulp of the reference), lse 1e-3; fp32 inputs ->
1e-4; rows that see no key -> exactly 0 and -inf.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_inputs, workload
from parity import compare, oracle_rows, run_gpu

pytestmark = pytest.mark.gpu


def _full_compare(cfg, out_dtype, use_subtiling=False, scale=None):
    q, k, v = make_inputs(cfg)
    in_dt = cfg["dtype"]
    od = {"bf16": torch.bfloat16, "fp32": torch.float32}[out_dtype]
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=od, lse=True, use_subtiling=use_subtiling,
                          scale=scale)
    ref_out, ref_lse = oracle_rows(cfg, q, k, v, scale=scale)
    D = cfg["d"]
    return compare(out.reshape(-1, D), lse.reshape(-1), ref_out, ref_lse, in_dt, out_dtype,
                   what=cfg["name"])


# Reduced versions of each workload: several tiles in both directions and a
# ragged tail in both lengths.
SMALL = [
    ("tiny_causal", {}),
    ("tiny_causal", dict(q_len=200, kv_len=200)),
    ("tiny_causal", dict(q_block=128, kv_block=128, q_len=300, kv_len=300, d=128)),
    ("prefix_causal", dict(B=1, H=2, q_len=1000, kv_len=1000, mask={"kind": "prefix_causal", "prefix": 300})),
    ("prefix_causal", dict(B=2, H=1, q_len=520, kv_len=520, mask={"kind": "prefix_causal", "prefix": 256})),
    ("sliding_window", dict(B=1, H=2, q_len=1100, kv_len=1100)),
    ("sliding_window", dict(B=1, H=1, q_len=700, kv_len=700, mask={"kind": "sliding_window", "window": 100, "window_min": 3})),
    ("long_causal_d128", dict(B=1, H=2, q_len=777, kv_len=777)),
    ("long_causal_d128", dict(B=1, H=2, q_len=300, kv_len=300, q_block=64, kv_block=64)),
    ("causal_rel_bias", dict(B=1, H=8, q_len=700, kv_len=700)),
    ("causal_rel_bias", dict(B=1, H=3, q_len=333, kv_len=333, q_block=128, kv_block=64)),
    ("prefix_causal", dict(B=1, H=2, q_len=300, kv_len=650, mask={"kind": "noop"})),
    ("prefix_causal", dict(B=1, H=1, q_len=650, kv_len=300, mask={"kind": "causal"}, q_block=64, kv_block=64)),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_small_parity(name, over, out_dtype):
    cfg = workload(name, **over)
    if "d" in over:
        cfg["scale"] = fa.default_scale(cfg["d"])
    _full_compare(cfg, out_dtype)


def test_small_parity_subtiling():
    cfg = workload("sliding_window", B=1, H=2, q_len=1100, kv_len=1100)
    _full_compare(cfg, "fp32", use_subtiling=True)


def test_negative_scale():
    cfg = workload("prefix_causal", B=1, H=1, q_len=300, kv_len=300)
    _full_compare(cfg, "fp32", scale=-0.2)


def test_fp32_rel_bias_and_window():
    cfg = workload("tiny_causal", H=4, mask={"kind": "sliding_window", "window": 50},
                   score={"kind": "rel_bias", "bias_max": 8.0})
    _full_compare(cfg, "fp32")


# ---- full-size workloads in the benchmark's launch configuration ----


@pytest.mark.parametrize("name", ["prefix_causal", "sliding_window", "long_causal_d128",
                                  "causal_rel_bias"])
def test_full_size_every_row(name):
    """The full workload, every one of its B*H*Lq rows against the oracle
    (run on every host core), with bf16 output (what the benchmark stores)
    and fp32 output; prints the raw largest errors of out and lse."""
    cfg = workload(name)
    q, k, v = make_inputs(cfg)
    D = cfg["d"]
    ref_out, ref_lse = oracle_rows(cfg, q, k, v)
    for out_dtype in ("bf16", "fp32"):
        od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=od, lse=True)
        e_out, e_lse = compare(out.reshape(-1, D), lse.reshape(-1), ref_out, ref_lse, "bf16",
                               out_dtype, what=name + "/" + out_dtype)
        print("\nfull-size %s, %s output, %d rows: max |out - ref| = %.3e, max |lse - ref| = %.3e"
              % (name, out_dtype, ref_lse.shape[0], e_out, e_lse), flush=True)


def test_full_size_tiny_causal():
    _full_compare(workload("tiny_causal"), "fp32")


# ---- invariants that hold bit for bit ----


def _bitwise(a, b):
    return np.array_equal(a.view(np.uint64), b.view(np.uint64)) if a.dtype == np.float64 else np.array_equal(a, b)


def test_subtiling_is_bitwise_identical():
    cfg = workload("sliding_window")
    q, k, v = make_inputs(cfg)
    o0, l0, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True, use_subtiling=False)
    o1, l1, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True, use_subtiling=True)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("name", ["prefix_causal", "sliding_window", "document_causal"])
def test_reruns_are_deterministic(name):
    """The full workload four times on the same inputs and block mask: every
    run bitwise equal (work-groups share nothing but LDS within a group, so
    a difference means a missing wait or barrier)."""
    cfg = workload(name)
    q, k, v = make_inputs(cfg)
    dev = torch.device("cuda:0")
    from block_sparse_masked_flexattention_amd.inputs import with_doc_ids
    mask = with_doc_ids(cfg, dev)
    bm = fa.build_block_mask(mask, cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"],
                             device=dev)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    runs = []
    for _ in range(4):
        o, l = fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], out_dtype=torch.float32,
                      return_lse=True)
        runs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for o, l in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])


def _demoted(bm, with_empty):
    """Same visiting order, but every full tile listed as partial (and, with
    with_empty, every empty tile listed as partial too).  The kernel walks
    the partial list from its last entry down, then the full list the same
    way, so the demoted list is empty + full + partial."""
    kvn, kvi, fkn, fki = (a.cpu() for a in bm.arrays())
    nq, nk = kvi.shape
    n_kvi = torch.zeros_like(kvi)
    n_kvn = torch.zeros_like(kvn)
    for qb in range(nq):
        lst = [int(x) for x in fki[qb, :fkn[qb]]] + [int(x) for x in kvi[qb, :kvn[qb]]]
        if with_empty:
            lst = [kb for kb in range(nk) if kb not in set(lst)] + lst
        rest = [kb for kb in range(nk) if kb not in set(lst)]
        n_kvi[qb] = torch.tensor(lst + rest, dtype=torch.int32)
        n_kvn[qb] = len(lst)
    dev = bm.kv_indices.device
    return fa.BlockMask(bm.mask, bm.q_len, bm.kv_len, bm.q_block, bm.kv_block,
                        n_kvn.to(dev), n_kvi.to(dev), torch.zeros_like(bm.full_kv_num_blocks),
                        bm.full_kv_indices.clone())


DEMOTE = [
    ("prefix_causal", dict(B=1, H=2, q_len=1024, kv_len=1024, mask={"kind": "prefix_causal", "prefix": 300})),
    ("causal_rel_bias", dict(B=1, H=8, q_len=512, kv_len=512)),
    ("long_causal_d128", dict(B=1, H=2, q_len=512, kv_len=512)),
]


@pytest.mark.parametrize("name,over", DEMOTE)
def test_full_tiles_demoted_to_partial_are_bitwise_equal(name, over):
    """Full tiles listed as partial: the same tiles in the same order, the
    mask evaluated on them and found to hide nothing, so the result is
    bitwise the same."""
    cfg = workload(name, **over)
    q, k, v = make_inputs(cfg)
    o0, l0, bm = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    o1, l1, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True,
                        bm=_demoted(bm, with_empty=False))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("name,over", DEMOTE)
def test_empty_tiles_listed_as_partial(name, over):
    """Every empty tile listed as partial too: each is visited and, block by
    block, skipped, so the result is the same softmax.  It is not always
    the same bits: listed empty tiles can come first in the walk, and then
    a row's first keys come through the fast path's fallback rather than
    the exact first step, so the offset its later probabilities are rounded
    to bf16 against can differ (out within the bf16 rounding of p, lse
    within fp32 rounding).  Both results meet the oracle bars."""
    cfg = workload(name, **over)
    q, k, v = make_inputs(cfg)
    o0, l0, bm = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    o1, l1, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True,
                        bm=_demoted(bm, with_empty=True))
    assert np.abs(o0 - o1).max() <= 4e-3 and np.abs(l0 - l1).max() <= 1e-5
    ref_out, ref_lse = oracle_rows(cfg, q, k, v)
    D = cfg["d"]
    compare(o1.reshape(-1, D), l1.reshape(-1), ref_out, ref_lse, "bf16", "fp32",
            what=name + " empty tiles listed")


def test_causal_row0_returns_v0_exactly():
    cfg = workload("prefix_causal", B=1, H=2, q_len=256, kv_len=256, mask={"kind": "causal"})
    q, k, v = make_inputs(cfg)
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    np.testing.assert_array_equal(out[:, :, 0, :], v[:, :, 0, :].double().numpy())
    s00 = (q[:, :, 0, :].double() * k[:, :, 0, :].double()).sum(-1) * cfg["scale"]
    np.testing.assert_allclose(lse[:, :, 0], s00.numpy(), atol=1e-5)


def test_uniform_scores_closed_form():
    """q = 0: every visible key weighs the same, lse = ln(count)."""
    cfg = workload("sliding_window", B=1, H=1, q_len=600, kv_len=600,
                   mask={"kind": "sliding_window", "window": 130})
    q, k, v = make_inputs(cfg)
    q = torch.zeros_like(q)
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    i = np.arange(600)
    count = np.minimum(i, 130) + 1
    np.testing.assert_allclose(lse[0, 0], np.log(count), atol=1e-5)
    vv = v[0, 0].double().numpy()
    csum = np.concatenate([np.zeros((1, vv.shape[1])), np.cumsum(vv, 0)])
    mean = (csum[i + 1] - csum[i + 1 - count]) / count[:, None]
    np.testing.assert_allclose(out[0, 0], mean, atol=1e-5)


# ---- degenerate shapes ----


def test_fully_masked_rows_and_blocks():
    # window_min = 200 > 0: rows 0..199 see nothing; with 128-row q-blocks the
    # first q-block has no tile at all
    cfg = workload("sliding_window", B=1, H=2, q_len=520, kv_len=520,
                   mask={"kind": "sliding_window", "window": 300, "window_min": 200})
    max_out, _ = _full_compare(cfg, "fp32")
    q, k, v = make_inputs(cfg)
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    assert np.all(np.isneginf(lse[:, :, :200])) and np.all(out[:, :, :200] == 0)


def test_no_keys():
    cfg = workload("prefix_causal", B=1, H=2, q_len=130, kv_len=0)
    q, k, v = make_inputs(cfg)
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_no_queries_and_no_batch():
    for over in (dict(q_len=0), dict(B=0)):
        cfg = workload("prefix_causal", H=2, kv_len=256, **({"q_len": 256} | over))
        q, k, v = make_inputs(cfg)
        out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
        assert out.size == 0 and lse.size == 0


def test_single_row_single_key():
    cfg = workload("tiny_causal", q_len=1, kv_len=1)
    q, k, v = make_inputs(cfg)
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    np.testing.assert_array_equal(out[0, 0, 0], v[0, 0, 0].double().numpy())
    assert math.isfinite(float(lse[0, 0, 0]))


def _with_direction(cfg, key_col0, q_col0=1.0):
    """The workload's inputs with q[..., 0] = q_col0 and k[..., 0] set from
    key_col0 (a function of the key index), stored in the workload dtype."""
    q, k, v = make_inputs(cfg)
    dt = q.dtype
    qf, kf = q.float().clone(), k.float().clone()
    qf[..., 0] = q_col0
    kf[..., 0] = key_col0(torch.arange(cfg["kv_len"], dtype=torch.float32))
    return qf.to(dt).contiguous(), kf.to(dt).contiguous(), v


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("trend", [4.0, -4.0])
@pytest.mark.parametrize("mask", [{"kind": "causal"},
                                  {"kind": "sliding_window", "window": 150, "window_min": 0}])
def test_monotone_score_trend(dtype, trend, mask):
    """Scores that rise (or fall) by about 23 log2 units per 32 keys.  Rising,
    nearly every block raises the row's offset (the kernel's rescale path);
    falling, later probabilities underflow to zero.  Same tolerances as the
    other parity tests."""
    cfg = workload("tiny_causal", B=1, H=2, q_len=333, kv_len=333, dtype=dtype, mask=mask)
    q, k, v = _with_direction(cfg, lambda j: trend * j)
    for od in ("fp32", "bf16"):
        out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=getattr(torch, {"fp32": "float32", "bf16": "bfloat16"}[od]),
                              lse=True)
        ref_out, ref_lse = oracle_rows(cfg, q, k, v)
        compare(out.reshape(-1, cfg["d"]), lse.reshape(-1), ref_out, ref_lse, dtype, od,
                what="trend %g %s %s" % (trend, mask["kind"], od))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_score_spike_mid_row(dtype):
    """One key (index 150) scores about 72 log2 units above every other key
    of a row: rows that reach it switch their offset there, mid-row and
    mid-tile."""
    cfg = workload("prefix_causal", B=1, H=2, q_len=400, kv_len=400, dtype=dtype,
                   mask={"kind": "causal"}, q_block=128, kv_block=64)
    q, k, v = _with_direction(cfg, lambda j: torch.where(j == 150, 400.0, 0.0))
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.float32, lse=True)
    ref_out, ref_lse = oracle_rows(cfg, q, k, v)
    compare(out.reshape(-1, cfg["d"]), lse.reshape(-1), ref_out, ref_lse, dtype, "fp32",
            what="spike")
    # rows past the spike return v[150] up to the tolerance
    o = out.reshape(cfg["B"], cfg["H"], cfg["q_len"], cfg["d"])
    vf = v.double().numpy()
    tol = 1e-2 if dtype == "bf16" else 1e-4
    assert np.abs(o[:, :, 150:, :] - vf[:, :, 150:151, :]).max() <= tol


@pytest.mark.parametrize("kv_block", [64, 128])
def test_many_items_per_workgroup(kv_block):
    """2048 (head, q-block) work-groups, several times what the chip holds at
    once, each with a short tile list; kv_block 64 gives odd step counts,
    128 even ones.  Every row is compared."""
    cfg = workload("prefix_causal", B=16, H=64, q_len=200, kv_len=200,
                   mask={"kind": "prefix_causal", "prefix": 70}, q_block=128, kv_block=kv_block)
    _full_compare(cfg, "fp32")


def test_items_without_tiles_between_full_ones():
    """5120 (head, q-block) work items, several times what the device holds
    at once: every fifth q-block (the first of each head) has no tile at all
    (window_min 200 > its last row), so empty items sit between full ones
    in the dispatch order.  Every row is compared; the empty rows are
    exactly 0 and -inf."""
    cfg = workload("sliding_window", B=16, H=64, q_len=520, kv_len=520,
                   mask={"kind": "sliding_window", "window": 300, "window_min": 200})
    _full_compare(cfg, "fp32")
    q, k, v = make_inputs(cfg)
    out, lse, _ = run_gpu(cfg, q, k, v, out_dtype=torch.bfloat16, lse=True)
    assert np.all(np.isneginf(lse[:, :, :200])) and np.all(out[:, :, :200] == 0)


def test_many_items_head_dim_128():
    """Head dim 128 (two waves per SIMD, so fewer resident work-groups) with
    many more short items than resident work-groups, and ragged lengths."""
    cfg = workload("long_causal_d128", B=8, H=32, q_len=333, kv_len=333)
    _full_compare(cfg, "bf16")


@pytest.mark.parametrize("name,over", [
    ("prefix_causal", dict(B=2, H=2, q_len=333, kv_len=333, mask={"kind": "prefix_causal", "prefix": 100})),
    ("sliding_window", dict(B=1, H=3, q_len=461, kv_len=461)),
    ("long_causal_d128", dict(B=1, H=2, q_len=297, kv_len=297)),
    ("prefix_causal", dict(B=1, H=2, q_len=201, kv_len=201, dv=128, mask={"kind": "causal"})),
])
def test_bf16_out_rows_stay_inside_the_tensor(name, over):
    """bf16 output of ragged lengths (the q-block past the last row still
    runs): every row matches the oracle and nothing past the end of the
    output tensor is written."""
    cfg = workload(name, **over)
    q, k, v = make_inputs(cfg)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    B, H, Lq, Dv = cfg["B"], cfg["H"], cfg["q_len"], cfg.get("dv", cfg["d"])
    n = B * H * Lq * Dv
    pad = 64 * 1024
    sentinel = -12345.0  # exact in bf16
    flat = torch.full((n + pad,), sentinel, dtype=torch.bfloat16, device=dev)
    out = flat[:n].view(B, H, Lq, Dv)
    bm = fa.build_block_mask(cfg["mask"], Lq, cfg["kv_len"], cfg["q_block"], cfg["kv_block"], device=dev)
    fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], out=out)
    torch.cuda.synchronize()
    assert bool((flat[n:] == sentinel).all()), "write past the end of the output"
    ref_out, ref_lse = oracle_rows(cfg, q, k, v)
    compare(out.double().cpu().numpy().reshape(-1, Dv), None, ref_out, ref_lse, "bf16", "bf16",
            what=name)


def test_binding_refuses_host_tensors_beside_gpu_inputs():
    """GPU q/k/v with a host output, lse or block mask is refused with
    ValueError before the library is called (such a pointer would reach a
    kernel as a host address)."""
    cfg = workload("prefix_causal", B=1, H=1, q_len=256, kv_len=256)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(cfg))
    bm = fa.build_block_mask(cfg["mask"], 256, 256, 128, 64, device=dev)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, bm, out=torch.empty(1, 1, 256, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, bm, lse=torch.empty(1, 1, 256))
    host_bm = fa.BlockMask(bm.mask, 256, 256, 128, 64, *[a.cpu() for a in bm.arrays()])
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, host_bm)
    short_bm = fa.BlockMask(bm.mask, 256, 256, 128, 64, bm.kv_num_blocks[:1].contiguous(),
                            bm.kv_indices, bm.full_kv_num_blocks, bm.full_kv_indices)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, short_bm)
    out, _ = fa.fwd(q, k, v, bm)  # and the well-formed call still runs
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
