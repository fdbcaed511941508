"""Pins for the oracle's row max (the OUTPUT_MAX output of the flex_attention
op in the test hunks of "[Inductor][Flex Attention] Add Subtiling Option for
Alpha Scaling"): closed forms the relative bias gives with q = 0, single-key
and fully masked rows, a two-key worked example, and the bounds that tie the
max to the log-sum-exp (max <= lse <= max + ln(count), equality on the right
exactly for uniform scores)."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle


def _rand(shape, seed, std=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).numpy()


def _count(mask, i, kv_len):
    """Keys row i sees, by the element predicate written out."""
    kind = mask["kind"]
    n = 0
    for j in range(kv_len):
        if kind == "noop":
            ok = True
        elif kind == "causal":
            ok = i >= j
        elif kind == "sliding_window":
            ok = mask.get("window_min", 0) <= i - j <= mask["window"]
        else:
            P = mask["prefix"]
            ok = (i <= P and j <= P) or i >= j
        n += ok
    return n


MASKS = [{"kind": "noop"}, {"kind": "causal"},
         {"kind": "sliding_window", "window": 5, "window_min": 2},
         {"kind": "prefix_causal", "prefix": 9}]


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m["kind"])
def test_uniform_scores_max_is_zero(mask):
    """q = 0: every visible score is 0, so the max is 0 (and lse = ln count);
    rows that see nothing get -inf."""
    L, D = 24, 8
    q = np.zeros((1, 1, L, D), np.float32)
    k = _rand((1, 1, L, D), 3)
    v = _rand((1, 1, L, D), 4)
    _, lse, mx = oracle.attention_rows(q, k, v, mask, {"kind": "identity"}, 0.7, with_max=True)
    for i in range(L):
        c = _count(mask, i, L)
        if c == 0:
            assert mx[i] == -math.inf and lse[i] == -math.inf
        else:
            assert mx[i] == 0.0
            assert abs(lse[i] - math.log(c)) < 1e-12


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m["kind"])
def test_rel_bias_max_is_the_nearest_visible_key(mask):
    """q = 0 with the relative bias: s_ij = -slope_h (i - j), largest at the
    largest visible j.  causal: 0; window_min w: -slope w; prefix P with
    i <= P: keys up to P are visible, so +slope (P - i); no mask: j = L-1."""
    H, L, D = 4, 24, 8
    q = np.zeros((1, H, L, D), np.float32)
    k = _rand((1, H, L, D), 5)
    v = _rand((1, H, L, D), 6)
    _, _, mx = oracle.attention_rows(q, k, v, mask, {"kind": "rel_bias", "bias_max": 8.0}, 1.0,
                                     with_max=True)
    mx = mx.reshape(H, L)
    for h in range(H):
        slope = 2.0 ** (-8.0 * (h + 1) / H)
        for i in range(L):
            kind = mask["kind"]
            if kind == "noop":
                want = -slope * (i - (L - 1))
            elif kind == "causal":
                want = 0.0
            elif kind == "sliding_window":
                w = mask["window_min"]
                want = -slope * w if i >= w else -math.inf
            else:
                P = mask["prefix"]
                want = slope * (P - i) if i <= P else 0.0
            if want == -math.inf:
                assert mx[h, i] == -math.inf
            else:
                assert abs(mx[h, i] - want) < 1e-14, (h, i, mx[h, i], want)


def test_two_key_worked_example_and_single_key_rows():
    # row 1 of a causal mask sees keys 0 and 1 with scores 0.5*1*2 = 1 and
    # 0.5*1*(-4) = -2: max 1.  Row 0 sees one key: max = lse = its score.
    q = np.array([[[[1.0, 0.0], [1.0, 0.0]]]], np.float32)
    k = np.array([[[[2.0, 0.0], [-4.0, 0.0]]]], np.float32)
    v = np.zeros((1, 1, 2, 2), np.float32)
    _, lse, mx = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "identity"}, 0.5,
                                       with_max=True)
    assert mx[0] == 1.0 and lse[0] == 1.0
    assert mx[1] == 1.0
    assert abs(lse[1] - math.log(math.exp(1.0) + math.exp(-2.0))) < 1e-15


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m["kind"])
@pytest.mark.parametrize("score", [{"kind": "identity"}, {"kind": "rel_bias", "bias_max": 8.0}],
                         ids=["identity", "rel_bias"])
def test_max_lse_bounds(mask, score):
    """Random inputs: max <= lse <= max + ln(count), strict on both sides
    unless the row has one key."""
    H, L, D = 2, 30, 16
    q, k, v = _rand((1, H, L, D), 7), _rand((1, H, L, D), 8), _rand((1, H, L, D), 9)
    _, lse, mx = oracle.attention_rows(q, k, v, mask, score, 0.25, with_max=True)
    lse, mx = lse.reshape(H, L), mx.reshape(H, L)
    for h in range(H):
        for i in range(L):
            c = _count(mask, i, L)
            if c == 0:
                assert mx[h, i] == -math.inf
                continue
            if c == 1:
                assert mx[h, i] == lse[h, i]
                continue
            assert mx[h, i] < lse[h, i] < mx[h, i] + math.log(c)


def test_max_is_optional_and_leaves_outputs_unchanged():
    q, k, v = _rand((1, 2, 20, 8), 10), _rand((1, 2, 20, 8), 11), _rand((1, 2, 20, 8), 12)
    a = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "identity"}, 0.3)
    b = oracle.attention_rows(q, k, v, {"kind": "causal"}, {"kind": "identity"}, 0.3, with_max=True)
    assert len(a) == 2 and len(b) == 3
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
