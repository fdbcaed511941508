"""Pins of the fp64 oracle's backward and transposed block arrays (CPU only).

The backward of the oracle (``oracle_attention_backward``) is the chain rule
written out by hand.  It is checked against things it does not share code
with:
  * central finite differences of the oracle's *forward* (a separate routine)
    through the loss  L = <out, dout> + <lse, dlse>;
  * torch autograd in fp64: of ``scaled_dot_product_attention`` (a library
    routine) for the mask kinds it expresses as a boolean mask, and of the
    masked-softmax forward for the relative bias;
  * closed forms: with q = 0 every visible weight is 1 / count_i, so
    dv_j = sum over rows i that see j of dout_i / count_i; and the softmax
    gradient of a row sums to dlse_i, so sum_j dk_j = scale * sum_i dlse_i q_i;
  * a fully masked row contributes nothing and gets dq = 0.
The transposed block arrays are checked against the (already pinned)
kv-major arrays tile by tile, and on a hand-worked case.
"""
import numpy as np
import pytest
import torch

from oracle import oracle

MASKS = [
    {"kind": "noop"},
    {"kind": "causal"},
    {"kind": "sliding_window", "window": 5, "window_min": 0},
    {"kind": "prefix_causal", "prefix": 4},
]


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("mask", MASKS, ids=[m["kind"] for m in MASKS])
@pytest.mark.parametrize("score", [{"kind": "identity"}, {"kind": "rel_bias", "bias_max": 8.0},
                                   {"kind": "rel_bias", "slopes": np.array([0.9, -0.4], np.float32)}],
                         ids=["identity", "rel_bias", "slope_table"])
def test_backward_matches_finite_differences(mask, score):
    B, H, Lq, Lk, D, Dv = 1, 2, 9, 11, 4, 3
    q, k, v = _rand((B, H, Lq, D), 1), _rand((B, H, Lk, D), 2), _rand((B, H, Lk, Dv), 3)
    dout, dlse = _rand((B, H, Lq, Dv), 4), _rand((B, H, Lq), 5)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, mask, score, scale, dlse=dlse)
    # central differences of the loss with fp64 inputs (a perturbation of
    # 1e-3 would be rounded by float32)
    eps = 1e-3
    rng = np.random.default_rng(6)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            vals = []
            for sgn in (1, -1):
                a = arr.astype(np.float64).copy()
                a[idx] += sgn * eps
                args = {"q": q, "k": k, "v": v}
                args[name] = a
                vals.append(_loss64(args["q"], args["k"], args["v"], dout, dlse, mask, score, scale))
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def _loss64(q, k, v, dout, dlse, mask, score, scale):
    """The same loss with fp64 inputs, by a dense numpy forward (independent of
    the C oracle), so a perturbation of 1e-3 is not rounded to float32."""
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    kind = mask["kind"]
    if kind == "noop":
        m = np.ones((Lq, Lk), bool)
    elif kind == "causal":
        m = i >= j
    elif kind == "sliding_window":
        m = (i - j >= mask.get("window_min", 0)) & (i - j <= mask["window"])
    else:
        P = mask["prefix"]
        m = ((i <= P) & (j <= P)) | (i >= j)
    total = 0.0
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T)
            if score.get("kind") == "rel_bias":
                slope = float(score["slopes"][h]) if "slopes" in score else \
                    2.0 ** (-score["bias_max"] * (h + 1) / H)
                s = s - slope * (i - j)
            s = np.where(m, s, -np.inf)
            for r in range(Lq):
                if not m[r].any():
                    continue
                mx = s[r].max()
                w = np.exp(s[r] - mx)
                l = w.sum()
                out = (w[:, None] * v[b, h].astype(np.float64)).sum(0) / l
                total += float(out @ dout[b, h, r]) + float((mx + np.log(l)) * dlse[b, h, r])
    return total


def _torch_mask(mask, Lq, Lk):
    i = torch.arange(Lq)[:, None]
    j = torch.arange(Lk)[None, :]
    kind = mask["kind"]
    if kind == "noop":
        return torch.ones(Lq, Lk, dtype=torch.bool)
    if kind == "causal":
        return i >= j
    if kind == "sliding_window":
        return (i - j >= mask.get("window_min", 0)) & (i - j <= mask["window"])
    P = mask["prefix"]
    return ((i <= P) & (j <= P)) | (i >= j)


@pytest.mark.parametrize("mask", MASKS, ids=[m["kind"] for m in MASKS])
def test_backward_matches_torch_sdpa_autograd(mask):
    """Every row sees at least one key (Lq <= Lk, diagonal visible), so SDPA
    is defined on all rows; dlse = 0 (SDPA returns no lse)."""
    B, H, Lq, Lk, D = 2, 3, 17, 17, 8
    q, k, v = _rand((B, H, Lq, D), 11), _rand((B, H, Lk, D), 12), _rand((B, H, Lk, D), 13)
    dout = _rand((B, H, Lq, D), 14)
    scale = 0.3
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, mask, {"kind": "identity"}, scale)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=_torch_mask(mask, Lq, Lk), scale=scale)
    out.backward(torch.tensor(dout, dtype=torch.float64))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-10)


def test_backward_rel_bias_matches_torch_autograd():
    """Relative bias and an lse gradient: torch autograd of the masked-softmax
    forward (logsumexp and softmax from torch) in fp64."""
    B, H, Lq, Lk, D = 1, 4, 13, 13, 8
    q, k, v = _rand((B, H, Lq, D), 21), _rand((B, H, Lk, D), 22), _rand((B, H, Lk, D), 23)
    dout, dlse = _rand((B, H, Lq, D), 24), _rand((B, H, Lq), 25)
    scale = 0.35
    score = {"kind": "rel_bias", "bias_max": 8.0}
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, {"kind": "causal"}, score, scale,
                                           dlse=dlse)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    i = torch.arange(Lq)[:, None].double()
    j = torch.arange(Lk)[None, :].double()
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float64)
    s = scale * tq @ tk.transpose(-1, -2) - slopes[None, :, None, None] * (i - j)
    s = s.masked_fill(~(i >= j), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    out = torch.softmax(s, dim=-1) @ tv
    loss = (out * torch.tensor(dout, dtype=torch.float64)).sum() + \
        (lse * torch.tensor(dlse, dtype=torch.float64)).sum()
    loss.backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-10)


@pytest.mark.parametrize("mask", MASKS, ids=[m["kind"] for m in MASKS])
def test_uniform_scores_dv_closed_form(mask):
    B, H, Lq, Lk, D = 1, 1, 12, 12, 4
    q = np.zeros((B, H, Lq, D), np.float32)
    k, v = _rand((B, H, Lk, D), 31), _rand((B, H, Lk, D), 32)
    dout = _rand((B, H, Lq, D), 33)
    _, _, dv = oracle.attention_backward(q, k, v, dout, mask, {"kind": "identity"}, 1.0)
    vis = np.array([[oracle.mask_value(mask, i, j, Lq, Lk) for j in range(Lk)]
                    for i in range(Lq)])
    count = vis.sum(1)
    want = np.zeros((Lk, D))
    for i in range(Lq):
        for j in range(Lk):
            if vis[i, j]:
                want[j] += dout[0, 0, i] / count[i]
    np.testing.assert_allclose(dv[0, 0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", MASKS, ids=[m["kind"] for m in MASKS])
def test_dk_sums_to_lse_gradient_term(mask):
    B, H, Lq, Lk, D = 1, 2, 10, 10, 4
    q, k, v = _rand((B, H, Lq, D), 41), _rand((B, H, Lk, D), 42), _rand((B, H, Lk, D), 43)
    dout, dlse = _rand((B, H, Lq, D), 44), _rand((B, H, Lq), 45)
    scale = 0.5
    for dl in (None, dlse):
        _, dk, _ = oracle.attention_backward(q, k, v, dout, mask, {"kind": "identity"}, scale,
                                             dlse=dl)
        want = np.zeros((B, H, D)) if dl is None else \
            scale * np.einsum("bhi,bhid->bhd", dl.astype(np.float64), q.astype(np.float64))
        np.testing.assert_allclose(dk.sum(axis=2), want, rtol=0, atol=1e-11)


def test_fully_masked_row_gets_nothing():
    """window_min = 1: row 0 sees no key.  Its dq is 0 and its dout does not
    reach dk or dv."""
    mask = {"kind": "sliding_window", "window": 3, "window_min": 1}
    B, H, Lq, Lk, D = 1, 1, 8, 8, 4
    q, k, v = _rand((B, H, Lq, D), 51), _rand((B, H, Lk, D), 52), _rand((B, H, Lk, D), 53)
    dout = _rand((B, H, Lq, D), 54)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, mask, {"kind": "identity"}, 1.0)
    assert np.all(dq[0, 0, 0] == 0.0)
    dout2 = dout.copy()
    dout2[0, 0, 0] += 5.0
    _, dk2, dv2 = oracle.attention_backward(q, k, v, dout2, mask, {"kind": "identity"}, 1.0)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


SHAPES = [
    ({"kind": "causal"}, 256, 256, 64, 64),
    ({"kind": "prefix_causal", "prefix": 300}, 1000, 1000, 128, 64),
    ({"kind": "sliding_window", "window": 100, "window_min": 3}, 700, 700, 128, 128),
    ({"kind": "noop"}, 300, 650, 128, 64),
    ({"kind": "causal"}, 650, 300, 64, 64),
    ({"kind": "prefix_causal", "prefix": 1024}, 2048, 2048, 128, 64),
]


@pytest.mark.parametrize("mask,lq,lk,qb,kb", SHAPES)
def test_transposed_block_arrays_agree_with_kv_major(mask, lq, lk, qb, kb):
    kvn, kvi, fkn, fki = oracle.block_mask(mask, lq, lk, qb, kb)
    qn, qi, fqn, fqi = oracle.block_mask_t(mask, lq, lk, qb, kb)
    nq, nk = kvi.shape
    cls_rows = np.zeros((nq, nk), int)
    cls_cols = np.zeros((nq, nk), int)
    for r in range(nq):
        cls_rows[r, kvi[r, :kvn[r]]] = 1
        cls_rows[r, fki[r, :fkn[r]]] = 2
    for c in range(nk):
        cls_cols[qi[c, :qn[c]], c] = 1
        cls_cols[fqi[c, :fqn[c]], c] = 2
        # each column is a permutation of 0..nQB-1, selected blocks first and ascending
        assert sorted(qi[c]) == list(range(nq)) and sorted(fqi[c]) == list(range(nq))
        assert list(qi[c, :qn[c]]) == sorted(qi[c, :qn[c]])
        assert list(qi[c, qn[c]:]) == sorted(qi[c, qn[c]:])
    assert np.array_equal(cls_rows, cls_cols)


def test_transposed_block_arrays_hand_worked():
    """Causal, 4 x 4 keys in 2 x 2 tiles: tile (0,0) and (1,1) are partial
    (the diagonal), (1,0) is full, (0,1) is empty.  Column 0 sees q-block 0
    partial and q-block 1 full; column 1 sees q-block 1 partial."""
    qn, qi, fqn, fqi = oracle.block_mask_t({"kind": "causal"}, 4, 4, 2, 2)
    assert list(qn) == [1, 1] and list(fqn) == [1, 0]
    assert qi.tolist() == [[0, 1], [1, 0]]
    assert fqi.tolist() == [[1, 0], [0, 1]]
