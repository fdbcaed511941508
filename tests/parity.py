"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run
the oracle on the same inputs, compare under the stated tolerances.

Tolerances (also written in the tests that use them):
  * bf16 inputs, fp32 output: max |out - ref| <= 1e-2, max |lse - ref| <= 1e-3.
  * bf16 output (either input type): the bound above plus half a bf16 ulp of
    ref, since storing the result in bf16 alone moves it by that much.
  * fp32 inputs: out and lse within 1e-4 (fp32 products and sums over at most
    a few thousand terms of magnitude <= ~10).
  * rows that see no key: out exactly 0 and lse exactly -inf on both sides.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from oracle import oracle

TOL_BF16_OUT = 1e-2
TOL_BF16_LSE = 1e-3
TOL_FP32 = 1e-4


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -134)


def run_gpu(cfg, q, k, v, *, out_dtype=None, lse=None, use_subtiling=False, bm=None,
            scale=None):
    """Returns (out float64 numpy [B,H,Lq,D], lse numpy or None, block mask)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    want_lse = cfg.get("lse", False) if lse is None else lse
    if bm is None:
        bm = fa.build_block_mask(cfg["mask"], cfg["q_len"], cfg["kv_len"],
                                 cfg["q_block"], cfg["kv_block"], device=dev)
    out, l = fa.fwd(qd, kd, vd, bm, cfg.get("score"), cfg["scale"] if scale is None else scale,
                    out_dtype=out_dtype, return_lse=want_lse, use_subtiling=use_subtiling)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    return o, (l.double().cpu().numpy() if l is not None else None), bm


def oracle_rows(cfg, q, k, v, rows=None, scale=None):
    """fp64 oracle on the exact input values; rows = flat row ids or None."""
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    return oracle.attention_rows(qf, kf, vf, cfg["mask"], cfg.get("score", {"kind": "identity"}),
                                 cfg["scale"] if scale is None else scale, rows=rows)


def compare(out, lse, ref_out, ref_lse, in_dtype, out_dtype, what=""):
    """out [n, D] float64, lse [n] or None; ref from the oracle.  Returns the
    max errors for reporting."""
    assert out.shape == ref_out.shape, (out.shape, ref_out.shape)
    dead = np.isneginf(ref_lse)
    if lse is not None:
        assert np.array_equal(np.isneginf(lse), dead), what + ": -inf lse rows differ"
    if dead.any():
        assert np.all(out[dead] == 0.0), what + ": a fully masked row is not 0"
    live = ~dead
    err = np.abs(out - ref_out)
    max_out = float(err.max()) if err.size else 0.0
    max_lse = 0.0
    if lse is not None and live.any():
        max_lse = float(np.abs(lse[live] - ref_lse[live]).max())
    tol_out = TOL_FP32 if in_dtype == "fp32" else TOL_BF16_OUT
    tol_lse = TOL_FP32 if in_dtype == "fp32" else TOL_BF16_LSE
    if out_dtype == "fp32":
        assert max_out <= tol_out, "%s: out err %.3g > %g" % (what, max_out, tol_out)
    else:
        # a bf16 output is also rounded once more on store: half a bf16 ulp
        bound = tol_out + bf16_half_ulp(ref_out)
        worst = float((err - bound).max()) if err.size else -1.0
        assert worst <= 0.0, "%s: bf16 out err %.3g beyond %g + half ulp" % (what, max_out, tol_out)
    assert max_lse <= tol_lse, "%s: lse err %.3g > %g" % (what, max_lse, tol_lse)
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    return max_out, max_lse


def sample_rows(cfg, n_random=24, seed=0):
    """Flat row ids to check at full size: first/last rows, block and prefix
    boundaries, and random rows, over the first, last and a middle head."""
    B, H, L = cfg["B"], cfg["H"], cfg["q_len"]
    QB = cfg["q_block"]
    picks = {0, 1, QB - 1, QB, QB + 1, L // 2, L - QB, L - 2, L - 1}
    if cfg["mask"]["kind"] == "prefix_causal":
        P = cfg["mask"]["prefix"]
        picks |= {P - 1, P, P + 1}
    if cfg["mask"]["kind"] == "sliding_window":
        W = cfg["mask"]["window"]
        picks |= {W - 1, W, W + 1, W + QB}
    rng = np.random.default_rng(seed)
    picks |= set(int(x) for x in rng.integers(0, L, n_random))
    heads = sorted({0, B * H - 1, (B * H) // 2})
    rows = [bh * L + i for bh in heads for i in sorted(picks) if 0 <= i < L]
    return np.array(rows, dtype=np.int64)


def dtype_name(t: torch.dtype) -> str:
    return {torch.bfloat16: "bf16", torch.float32: "fp32"}[t]


def finite_or_neginf(x):
    return np.all(np.isfinite(x) | np.isneginf(x))


__all__ = ["run_gpu", "oracle_rows", "compare", "sample_rows", "dtype_name", "math"]
