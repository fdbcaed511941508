"""Pins for the fp64 oracle: checks against things other than the oracle itself.

* torch's fp64 CPU scaled_dot_product_attention (a library routine) for the
  unmasked and causal cases; the log-sum-exp is recovered from it through an
  extra "sink" key (see _sdpa_lse);
* closed forms for uniform scores (q = 0), including the geometric series a
  relative-position bias produces;
* single-key rows, fully masked rows;
* mask values the pages print, block arrays worked out by hand, and tile
  totals / per-row counts derived by interval reasoning for every workload.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, std=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).numpy()


def _sdpa_lse(q, k, v, scale):
    """LSE of unmasked attention from SDPA alone: append a key whose score is 0
    for every query and whose value is a one-hot extra column.  The output's
    extra column is exp(0 - LSE'), LSE' = log(exp(LSE) + 1)."""
    B, H, L, D = q.shape
    Dv = v.shape[-1]
    k2 = torch.cat([k, torch.zeros(B, H, 1, D, dtype=k.dtype)], dim=2)
    v2 = torch.cat([torch.cat([v, torch.zeros(B, H, L, 1, dtype=v.dtype)], -1),
                    torch.cat([torch.zeros(B, H, 1, Dv, dtype=v.dtype),
                               torch.ones(B, H, 1, 1, dtype=v.dtype)], -1)], dim=2)
    o2 = torch.nn.functional.scaled_dot_product_attention(q, k2, v2, scale=scale)
    lse_sink = -torch.log(o2[..., -1])
    return torch.log(torch.expm1(lse_sink))


# --------------------------------------------------------------------------
# softmax core against a library routine


@pytest.mark.parametrize("B,H,L,D,Dv", [(2, 3, 37, 16, 16), (1, 2, 64, 64, 32)])
def test_noop_matches_sdpa(B, H, L, D, Dv):
    q, k, v = _rand((B, H, L, D), 1), _rand((B, H, L, D), 2), _rand((B, H, L, Dv), 3)
    scale = 0.3
    out, lse = oracle.attention_rows(q, k, v, {"kind": "noop"}, {"kind": "identity"}, scale)
    tq, tk, tv = (torch.from_numpy(x).double() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    np.testing.assert_allclose(out.reshape(B, H, L, Dv), ref.numpy(), rtol=0, atol=1e-12)
    ref_lse = _sdpa_lse(tq, tk, tv, scale).numpy().reshape(-1)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-10)


def test_noop_rectangular_matches_sdpa():
    B, H, Lq, Lk, D = 1, 2, 19, 45, 8
    q, k, v = _rand((B, H, Lq, D), 4), _rand((B, H, Lk, D), 5), _rand((B, H, Lk, D), 6)
    out, _ = oracle.attention_rows(q, k, v, {"kind": "noop"}, {"kind": "identity"}, 0.7)
    tq, tk, tv = (torch.from_numpy(x).double() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.7)
    np.testing.assert_allclose(out.reshape(B, H, Lq, D), ref.numpy(), rtol=0, atol=1e-12)


def test_causal_matches_sdpa_is_causal():
    B, H, L, D = 2, 2, 70, 32
    q, k, v = _rand((B, H, L, D), 7), _rand((B, H, L, D), 8), _rand((B, H, L, D), 9)
    out, _ = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "identity"}, 0.125)
    tq, tk, tv = (torch.from_numpy(x).double() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.125)
    np.testing.assert_allclose(out.reshape(B, H, L, D), ref.numpy(), rtol=0, atol=1e-12)


def test_two_key_worked_example():
    # one query, two keys with scores 0 and ln 3 -> weights 1/4 and 3/4
    q = np.array([[[[1.0]]]], np.float32)
    k = np.array([[[[0.0], [1.0]]]], np.float32)
    v = np.array([[[[2.0, -4.0], [6.0, 8.0]]]], np.float32)
    out, lse = oracle.attention_rows(q, k, v, {"kind": "noop"}, {"kind": "identity"}, math.log(3.0))
    np.testing.assert_allclose(out[0], [0.25 * 2 + 0.75 * 6, 0.25 * -4 + 0.75 * 8], atol=1e-14)
    assert abs(lse[0] - math.log(4.0)) < 1e-14


# --------------------------------------------------------------------------
# uniform scores: q = 0, v[j, :] = j


def _visible_interval(mask, i, L):
    kind = mask["kind"]
    if kind == "noop":
        return 0, L - 1
    if kind == "causal":
        return 0, i
    if kind == "sliding_window":
        return max(0, i - mask["window"]), i - mask.get("window_min", 0)
    if kind == "prefix_causal":
        P = mask["prefix"]
        return 0, (max(P, i) if i <= P else i)
    raise ValueError(kind)


@pytest.mark.parametrize("mask", [
    {"kind": "noop"},
    {"kind": "causal"},
    {"kind": "sliding_window", "window": 5},
    {"kind": "sliding_window", "window": 9, "window_min": 3},
    {"kind": "prefix_causal", "prefix": 7},
])
def test_uniform_scores_closed_form(mask):
    L, D = 40, 4
    q = np.zeros((1, 1, L, D), np.float32)
    k = _rand((1, 1, L, D), 11)
    v = np.repeat(np.arange(L, dtype=np.float32)[None, None, :, None], 3, axis=3)
    out, lse = oracle.attention_rows(q, k, v, mask, {"kind": "identity"}, 0.9)
    for i in range(L):
        lo, hi = _visible_interval(mask, i, L)
        lo, hi = max(lo, 0), min(hi, L - 1)
        if hi < lo:
            assert lse[i] == -math.inf and np.all(out[i] == 0)
            continue
        count = hi - lo + 1
        assert abs(lse[i] - math.log(count)) < 1e-13
        np.testing.assert_allclose(out[i], (lo + hi) / 2.0, atol=1e-12)


@pytest.mark.parametrize("H", [8, 3])
def test_rel_bias_geometric_series(H):
    """q = 0, causal: weights r^(i-j) with r = exp(-slope_h); lse and the
    weighted mean of j have closed forms."""
    L, D = 50, 4
    q = np.zeros((1, H, L, D), np.float32)
    k = _rand((1, H, L, D), 12)
    v = np.repeat(np.arange(L, dtype=np.float32)[None, None, :, None], H, axis=1)
    out, lse = oracle.attention_rows(q, k, v, {"kind": "causal"},
                                     {"kind": "rel_bias", "bias_max": 8.0}, 1.0)
    out = out.reshape(H, L)
    lse = lse.reshape(H, L)
    for h in range(H):
        slope = 2.0 ** (-8.0 * (h + 1) / H)
        r = math.exp(-slope)
        for i in range(L):
            n = i  # terms t = i - j run over 0..n
            S = (1 - r ** (n + 1)) / (1 - r)
            T = r * (1 - (n + 1) * r ** n + n * r ** (n + 1)) / (1 - r) ** 2  # sum t r^t
            assert abs(lse[h, i] - math.log(S)) < 1e-12
            assert abs(out[h, i] - (i - T / S)) < 1e-10


@pytest.mark.parametrize("slopes", [[0.7, -0.3, 0.05], [1.5, 0.0, 2.0 ** -9]])
def test_slope_table_geometric_series(slopes):
    """A per-head slope table (a score_mod closing over a tensor): the same
    closed forms with r = exp(-slopes[h]), for any sign; a zero slope is
    the plain mean of the visible j."""
    H, L, D = len(slopes), 40, 4
    q = np.zeros((1, H, L, D), np.float32)
    k = _rand((1, H, L, D), 13)
    v = np.repeat(np.arange(L, dtype=np.float32)[None, None, :, None], H, axis=1)
    table = np.array(slopes, np.float32)
    out, lse = oracle.attention_rows(q, k, v, {"kind": "causal"},
                                     {"kind": "rel_bias", "slopes": table}, 1.0)
    out, lse = out.reshape(H, L), lse.reshape(H, L)
    for h in range(H):
        sl = float(table[h])
        for i in range(L):
            n = i
            if sl == 0.0:
                assert abs(lse[h, i] - math.log(n + 1)) < 1e-12
                assert abs(out[h, i] - i / 2.0) < 1e-10
                continue
            r = math.exp(-sl)
            S = (1 - r ** (n + 1)) / (1 - r)
            T = r * (1 - (n + 1) * r ** n + n * r ** (n + 1)) / (1 - r) ** 2
            assert abs(lse[h, i] - math.log(S)) < 1e-10 * max(1.0, abs(math.log(S)))
            assert abs(out[h, i] - (i - T / S)) < 1e-8


def test_slope_table_of_zeros_is_the_identity_score():
    B, H, L, D = 1, 3, 70, 8
    q, k, v = _rand((B, H, L, D), 14), _rand((B, H, L, D), 15), _rand((B, H, L, D), 16)
    a = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "identity"}, 0.3)
    b = oracle.attention_rows(q, k, v, {"kind": "causal"},
                              {"kind": "rel_bias", "slopes": np.zeros(H, np.float32)}, 0.3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_rel_bias_slopes_are_powers_of_two_for_8_heads():
    # with 8 heads slope_h = 2^-(h+1): a single-key row returns s_ii exactly and
    # a two-key row (j = i-1, i) has lse = log(e^{s_i,i-1 - slope} + e^{s_ii})
    H, L, D = 8, 2, 2
    q = np.ones((1, H, L, D), np.float32)
    k = np.zeros((1, H, L, D), np.float32)
    v = np.zeros((1, H, L, D), np.float32)
    _, lse = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "rel_bias"}, 1.0)
    lse = lse.reshape(H, L)
    for h in range(H):
        assert lse[h, 0] == 0.0
        assert abs(lse[h, 1] - math.log(math.exp(-(2.0 ** -(h + 1))) + 1.0)) < 1e-15


# --------------------------------------------------------------------------
# single-key and fully masked rows


def test_single_key_rows():
    L, D = 33, 16
    q, k, v = _rand((1, 1, L, D), 13), _rand((1, 1, L, D), 14), _rand((1, 1, L, D), 15)
    scale = 0.25
    out, lse = oracle.attention_rows(q, k, v, {"kind": "sliding_window", "window": 0},
                                     {"kind": "identity"}, scale)
    for i in range(L):
        np.testing.assert_array_equal(out[i], v[0, 0, i].astype(np.float64))
        s_ii = scale * float(np.dot(q[0, 0, i].astype(np.float64), k[0, 0, i].astype(np.float64)))
        assert abs(lse[i] - s_ii) < 1e-13
    # causal row 0 sees only key 0
    out_c, _ = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "identity"}, scale,
                                     rows=np.array([0]))
    np.testing.assert_array_equal(out_c[0], v[0, 0, 0].astype(np.float64))


def test_fully_masked_rows():
    L, D = 10, 8
    q, k, v = _rand((1, 1, L, D), 16), _rand((1, 1, L, D), 17), _rand((1, 1, L, D), 18)
    out, lse = oracle.attention_rows(q, k, v, {"kind": "sliding_window", "window": 3, "window_min": 1},
                                     {"kind": "identity"}, 0.5)
    assert lse[0] == -math.inf and np.all(out[0] == 0.0)
    assert np.all(np.isfinite(lse[1:]))
    # no keys at all
    k0 = np.zeros((1, 1, 0, D), np.float32)
    out0, lse0 = oracle.attention_rows(q, k0, k0, {"kind": "noop"}, {"kind": "identity"}, 0.5)
    assert np.all(lse0 == -math.inf) and np.all(out0 == 0.0)


# --------------------------------------------------------------------------
# mask values and block arrays


def test_prefix_mask_points_from_page():
    g = _golden("page_values.json")["prefix_causal_points"]
    mask = {"kind": "prefix_causal", "prefix": g["prefix"]}
    for p in g["points"]:
        assert oracle.mask_value(mask, p["q"], p["kv"], g["q_len"], g["kv_len"]) == p["visible"], p


def test_tiny_block_masks_by_hand():
    for case in _golden("tiny_block_mask.json")["cases"]:
        got = oracle.block_mask(case["mask"], case["q_len"], case["kv_len"],
                                case["q_block"], case["kv_block"])
        for name, arr in zip(["kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                              "full_kv_indices"], got):
            np.testing.assert_array_equal(arr, np.array(case[name], np.int32), err_msg=name)


def _interval_tiles(mask, q_len, kv_len, qb_size, kb_size):
    """Classify tiles from each row's visible interval (an independent route
    from element enumeration): full iff every row of the tile is in range and
    its interval covers the tile's columns; empty iff no row's interval meets
    them."""
    nq, nk = -(-q_len // qb_size), -(-kv_len // kb_size)
    cls = np.zeros((nq, nk), np.int8)
    for qb in range(nq):
        rows = range(qb * qb_size, min(q_len, (qb + 1) * qb_size))
        ivs = [_visible_interval(mask, i, kv_len) for i in rows]
        ivs = [(max(0, lo), min(kv_len - 1, hi)) for lo, hi in ivs]
        for kb in range(nk):
            c0, c1 = kb * kb_size, (kb + 1) * kb_size - 1
            any_vis = any(lo <= c1 and hi >= c0 and lo <= hi for lo, hi in ivs)
            full = (len(ivs) == qb_size and c1 < kv_len
                    and all(lo <= c0 and hi >= c1 for lo, hi in ivs))
            cls[qb, kb] = 2 if full else (1 if any_vis else 0)
    return cls


def _check_arrays_against_classes(arrs, cls):
    kvn, kvi, fkn, fki = arrs
    nq, nk = cls.shape
    for qb in range(nq):
        for want, num, idx in ((1, kvn, kvi), (2, fkn, fki)):
            sel = [kb for kb in range(nk) if cls[qb, kb] == want]
            rest = [kb for kb in range(nk) if cls[qb, kb] != want]
            assert num[qb] == len(sel)
            assert list(idx[qb]) == sel + rest


@pytest.mark.parametrize("mask,q_len,kv_len,qb,kb", [
    ({"kind": "causal"}, 300, 300, 64, 32),
    ({"kind": "causal"}, 97, 130, 16, 32),
    ({"kind": "noop"}, 45, 77, 16, 16),
    ({"kind": "sliding_window", "window": 40}, 260, 260, 32, 64),
    ({"kind": "sliding_window", "window": 17, "window_min": 5}, 129, 200, 16, 16),
    ({"kind": "prefix_causal", "prefix": 70}, 250, 250, 64, 32),
    ({"kind": "prefix_causal", "prefix": 63}, 128, 128, 32, 32),
])
def test_block_mask_matches_interval_reasoning(mask, q_len, kv_len, qb, kb):
    arrs = oracle.block_mask(mask, q_len, kv_len, qb, kb)
    _check_arrays_against_classes(arrs, _interval_tiles(mask, q_len, kv_len, qb, kb))


# Totals (full, partial) per (b, h) for each workload, from closed forms:
#  causal with n equal blocks: n(n-1)/2 full + n partial;
#  causal window 256 at 128x128 over 64 blocks: qb>=1 has one full tile
#  (kb = qb-1), qb>=2 two partial tiles (qb-2, qb), qb<=1 one partial;
#  prefix 1024 or causal at 128x64: qb 0-7 16 full + 1 partial, qb 8 16 + 2,
#  qb >= 9 2*qb full + 2 partial.
WORKLOAD_TILES = {
    "tiny_causal": (6, 4),
    "prefix_causal": (8 * 16 + 16 + sum(2 * q for q in range(9, 32)), 8 + 2 + 2 * 23),
    "sliding_window": (63, 1 + 1 + 2 * 62),
    "long_causal_d128": (128 * 127 // 2, 128),
    "causal_rel_bias": (256 * 255 // 2, 256),
}


@pytest.mark.parametrize("name", list(WORKLOAD_TILES))
def test_workload_tile_totals(name):
    from block_sparse_masked_flexattention_amd.inputs import workload
    cfg = workload(name)
    kvn, kvi, fkn, fki = oracle.block_mask(cfg["mask"], cfg["q_len"], cfg["kv_len"],
                                           cfg["q_block"], cfg["kv_block"])
    full, partial = WORKLOAD_TILES[name]
    assert int(fkn.sum()) == full and int(kvn.sum()) == partial
    nk = kvi.shape[1]
    for arr in (kvi, fki):  # every row is a permutation of the kv-blocks
        assert np.all(np.sort(arr, axis=1) == np.arange(nk)[None, :])
    if name == "prefix_causal":
        assert list(kvn) == [1] * 8 + [2] * 24
        assert list(fkn) == [16] * 9 + [2 * q for q in range(9, 32)]
    if name == "sliding_window":
        assert list(kvn) == [1, 1] + [2] * 62 and list(fkn) == [0] + [1] * 63


# visible (q, kv) pairs: the unmasked-FLOP count of the throughput metric
VISIBLE_PAIRS = {
    "tiny_causal": 256 * 257 // 2,
    "prefix_causal": 1025 * 1025 + (4096 * 4097 // 2 - 1025 * 1026 // 2),
    "sliding_window": 256 * 257 // 2 + (8192 - 256) * 257,
    "long_causal_d128": 16384 * 16385 // 2,
    "causal_rel_bias": 32768 * 32769 // 2,
}


@pytest.mark.parametrize("name", ["tiny_causal", "prefix_causal", "sliding_window"])
def test_visible_pairs_closed_form(name):
    from block_sparse_masked_flexattention_amd.inputs import workload
    cfg = workload(name)
    assert oracle.count_visible(cfg["mask"], cfg["q_len"], cfg["kv_len"]) == VISIBLE_PAIRS[name]


def test_default_scale_from_pages():
    from block_sparse_masked_flexattention_amd.inputs import default_scale
    for e in _golden("page_values.json")["default_scale"]:
        assert default_scale(e["head_dim"]) == e["scale"]
