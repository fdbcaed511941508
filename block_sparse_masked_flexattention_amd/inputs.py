"""Seeded synthetic workloads: shapes, mask and score settings, and inputs.

This module holds no attention arithmetic.  It only names the workloads
(tiny causal; prefix-bidirectional-or-causal; sliding window; long causal with
a 128-wide head; causal with a relative-position bias; packed documents,
causal inside each) and draws their q, k, v tensors (and document ids) from
seeded CPU generators, so the HIP path and the oracle read the exact same
values.

Recipe: ``torch.Generator("cpu").manual_seed(seed)``; q, k, v drawn in that
order with ``torch.randn(shape, float32)`` times ``std``; then rounded to
bfloat16 (round-to-nearest-even) unless the workload is float32.  Tensors are
contiguous ``[B, H, L, D]``.  The backward's output gradient (and the optional
log-sum-exp gradient) come from a second generator seeded ``seed + 7919``:
dout ~ N(0, 1) of q's shape and dtype, then dlse ~ N(0, 1) float32 [B, H, Lq].
"""
from __future__ import annotations

import math

import torch

WORKLOADS = {
    "tiny_causal": dict(
        B=1, H=1, q_len=256, kv_len=256, d=64, dtype="fp32", std=1.0,
        mask={"kind": "causal"}, score={"kind": "identity"},
        q_block=64, kv_block=64, lse=True, seed=1001,
    ),
    "prefix_causal": dict(
        B=4, H=16, q_len=4096, kv_len=4096, d=64, dtype="bf16", std=1.0,
        mask={"kind": "prefix_causal", "prefix": 1024}, score={"kind": "identity"},
        q_block=128, kv_block=64, lse=False, seed=1002,
    ),
    "sliding_window": dict(
        B=2, H=16, q_len=8192, kv_len=8192, d=64, dtype="bf16", std=1.0,
        mask={"kind": "sliding_window", "window": 256, "window_min": 0},
        score={"kind": "identity"},
        q_block=128, kv_block=128, lse=False, seed=1003,
    ),
    "long_causal_d128": dict(
        B=1, H=32, q_len=16384, kv_len=16384, d=128, dtype="bf16", std=1.0,
        mask={"kind": "causal"}, score={"kind": "identity"},
        q_block=128, kv_block=128, lse=True, seed=1004,
    ),
    "causal_rel_bias": dict(
        B=2, H=8, q_len=32768, kv_len=32768, d=64, dtype="bf16", std=0.5,
        mask={"kind": "causal"}, score={"kind": "rel_bias", "bias_max": 8.0},
        q_block=128, kv_block=128, lse=True, seed=1005,
    ),
    # packed sequences: documents of seeded random lengths, causal inside each
    "document_causal": dict(
        B=2, H=16, q_len=16384, kv_len=16384, d=64, dtype="bf16", std=1.0,
        mask={"kind": "document_causal"}, score={"kind": "identity"},
        q_block=128, kv_block=128, lse=False, seed=1006,
        doc_len_min=128, doc_len_max=3072,
    ),
}

# The workload the throughput benchmark runs by default.
BENCH_WORKLOAD = "prefix_causal"


def default_scale(d: int) -> float:
    """1/sqrt(head_dim) rounded to float32 (0.125 at d=64, 0.5 at d=4)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def workload(name: str, **overrides) -> dict:
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    cfg.setdefault("scale", default_scale(cfg["d"]))
    cfg["name"] = name
    return cfg


def doc_ids(cfg: dict, seed: int | None = None) -> torch.Tensor:
    """Per-token document ids (int32, CPU, non-decreasing) for a workload
    with a document mask: lengths drawn uniformly from [doc_len_min,
    doc_len_max] by a generator seeded ``seed + 104729`` until they cover the
    sequence; the last document is cut at the end.  Queries and keys share
    the ids (q_len == kv_len)."""
    g = torch.Generator("cpu").manual_seed((cfg["seed"] if seed is None else seed) + 104729)
    L = cfg["q_len"]
    lo, hi = cfg.get("doc_len_min", 1), cfg.get("doc_len_max", max(1, L))
    ids = torch.empty(L, dtype=torch.int32)
    pos, d = 0, 0
    while pos < L:
        n = int(torch.randint(lo, hi + 1, (1,), generator=g))
        ids[pos:pos + n] = d
        pos += n
        d += 1
    return ids


def with_doc_ids(cfg: dict, device=None) -> dict:
    """The workload's mask dict with q_doc / kv_doc filled in (on `device`)
    for a document mask; the mask unchanged otherwise."""
    mask = dict(cfg["mask"])
    if mask["kind"] in ("document", "document_causal"):
        if "q_doc" not in mask:
            mask["q_doc"] = mask["kv_doc"] = doc_ids(cfg)
        if device is not None:
            mask["q_doc"] = mask["q_doc"].to(device)
            mask["kv_doc"] = mask["kv_doc"].to(device)
    return mask


def make_inputs(cfg: dict, seed: int | None = None):
    """q, k, v as CPU tensors of the workload's dtype (bfloat16 or float32)."""
    g = torch.Generator("cpu").manual_seed(cfg["seed"] if seed is None else seed)
    B, H, Lq, Lk, D = cfg["B"], cfg["H"], cfg["q_len"], cfg["kv_len"], cfg["d"]
    dv = cfg.get("dv", D)
    std = cfg.get("std", 1.0)
    q = torch.randn((B, H, Lq, D), generator=g, dtype=torch.float32) * std
    k = torch.randn((B, H, Lk, D), generator=g, dtype=torch.float32) * std
    v = torch.randn((B, H, Lk, dv), generator=g, dtype=torch.float32) * std
    if cfg["dtype"] == "bf16":
        q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_grad_inputs(cfg: dict, with_dlse: bool = False, seed: int | None = None):
    """dout (the workload's dtype, q's shape) and dlse (float32 [B, H, Lq] or
    None) as CPU tensors, for the backward."""
    g = torch.Generator("cpu").manual_seed((cfg["seed"] if seed is None else seed) + 7919)
    B, H, Lq = cfg["B"], cfg["H"], cfg["q_len"]
    dv = cfg.get("dv", cfg["d"])
    dout = torch.randn((B, H, Lq, dv), generator=g, dtype=torch.float32)
    dlse = torch.randn((B, H, Lq), generator=g, dtype=torch.float32) if with_dlse else None
    if cfg["dtype"] == "bf16":
        dout = dout.to(torch.bfloat16)
    return dout.contiguous(), dlse
