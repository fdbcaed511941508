"""Seeded random sweep of the forward against the fp64 oracle: mask kind and
its parameters, score modification, head dims, tile shape, ragged and unequal
lengths, output dtype and the subtiled rescale are drawn per case, so that
combinations the hand-picked cases miss still meet the bar (bf16 inputs:
max-abs 1e-2 on the output, 1e-3 on the log-sum-exp; fp32 inputs: the fp32
bar of tests/parity.py on both)."""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd.inputs import make_inputs, with_doc_ids, workload
from parity import compare, oracle_rows, run_gpu

pytestmark = pytest.mark.gpu

HEAD_DIMS = [(64, 64), (128, 128), (64, 128), (128, 64)]
TILES = [(64, 64), (128, 64), (128, 128)]


def _case(seed):
    r = np.random.default_rng(7000 + seed)
    d, dv = HEAD_DIMS[r.integers(len(HEAD_DIMS))]
    qb, kb = TILES[r.integers(len(TILES))]
    kind = ["noop", "causal", "sliding_window", "prefix_causal", "document_causal"][r.integers(5)]
    lq = int(r.integers(1, 600))
    lk = lq if kind == "document_causal" else int(r.integers(1, 600))
    if kind == "sliding_window":
        mask = {"kind": kind, "window": int(r.integers(0, 300)), "window_min": int(r.integers(0, 3))}
    elif kind == "prefix_causal":
        mask = {"kind": kind, "prefix": int(r.integers(0, max(lq, 1)))}
    else:
        mask = {"kind": kind}
    score = {"kind": "rel_bias", "bias_max": 8.0} if r.integers(3) == 0 else {"kind": "identity"}
    H = int(r.integers(1, 4))
    over = dict(B=int(r.integers(1, 3)), H=H, q_len=lq, kv_len=lk, d=d, dv=dv, q_block=qb,
                kv_block=kb, mask=mask, score=score, seed=9000 + seed, doc_len_min=1,
                doc_len_max=int(r.integers(1, 300)))
    out_dtype = torch.bfloat16 if r.integers(2) else torch.float32
    return over, out_dtype, bool(r.integers(4) == 0)


def _run_case(seed, over, out_dtype, sub, in_dtype):
    cfg = workload("prefix_causal", **over)
    cfg["dtype"] = in_dtype
    cfg["mask"] = with_doc_ids(cfg)
    q, k, v = make_inputs(cfg)
    out, lse, _ = run_gpu(dict(cfg, mask=with_doc_ids(cfg, torch.device("cuda:0"))), q, k, v,
                          out_dtype=out_dtype, lse=True, use_subtiling=sub)
    ref_out, ref_lse = oracle_rows(cfg, q, k, v)
    compare(out.reshape(-1, cfg["dv"]), lse.reshape(-1), ref_out, ref_lse, in_dtype,
            "bf16" if out_dtype == torch.bfloat16 else "fp32",
            what="seed %d: %s" % (seed, {k_: over[k_] for k_ in ("q_len", "kv_len", "d", "dv", "q_block", "kv_block", "mask", "score")}))


@pytest.mark.parametrize("seed", range(64))
def test_random_case(seed):
    over, out_dtype, sub = _case(seed)
    _run_case(seed, over, out_dtype, sub, "bf16")


@pytest.mark.parametrize("seed", range(1000, 1024))
def test_random_case_fp32(seed):
    """The same draws with fp32 inputs (the fp32 kernel; the subtiling flag
    selects the same arithmetic there)."""
    over, out_dtype, sub = _case(seed)
    _run_case(seed, over, out_dtype, sub, "fp32")
