"""Pins for the oracle's document masks (a mask_mod closing over per-token
document ids, the op's mask_mod_other_buffers slot in the test hunks of
"[Inductor][Flex Attention] Add Subtiling Option for Alpha Scaling"):

* packed documents are independent sequences: every row equals torch's fp64
  scaled_dot_product_attention (a library routine) run on its document's
  slice alone, without a mask (document) or causal (document_causal); the
  log-sum-exp comes from the same routine through an extra zero-score key;
* any ids (unsorted, cross lengths): torch SDPA with the dense boolean mask
  q_doc[i] == kv_doc[j], and its autograd for the backward;
* one document is the no-mask / causal case (pinned elsewhere);
* block arrays worked out by hand.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).numpy()


def _sdpa_out_lse(q, k, v, scale, causal):
    """out and lse of [.., L, D] tensors by SDPA alone: an extra key with
    score 0 and a one-hot value column gives exp(-lse') in that column."""
    *lead, L, D = q.shape
    Lk, Dv = k.shape[-2], v.shape[-1]
    zk = torch.zeros(*lead, 1, D, dtype=k.dtype)
    k2 = torch.cat([k, zk], dim=-2)
    v2 = torch.cat([torch.cat([v, torch.zeros(*lead, Lk, 1, dtype=v.dtype)], -1),
                    torch.cat([torch.zeros(*lead, 1, Dv, dtype=v.dtype),
                               torch.ones(*lead, 1, 1, dtype=v.dtype)], -1)], dim=-2)
    i = torch.arange(L)[:, None]
    j = torch.arange(Lk + 1)[None, :]
    m = (j == Lk) | ((i >= j) if causal else torch.ones(L, Lk + 1, dtype=torch.bool))
    o2 = torch.nn.functional.scaled_dot_product_attention(q, k2, v2, attn_mask=m, scale=scale)
    lse_sink = -torch.log(o2[..., -1])
    out = o2[..., :-1] / (1.0 - o2[..., -1:])  # renormalise without the extra key
    return out, torch.log(torch.expm1(lse_sink))


@pytest.mark.parametrize("causal", [False, True])
def test_packed_documents_are_independent_sequences(causal):
    lens = [5, 1, 9, 3, 14]
    ids = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    L, D, H = int(ids.size), 8, 2
    q, k, v = _rand((1, H, L, D), 1), _rand((1, H, L, D), 2), _rand((1, H, L, D), 3)
    mask = {"kind": "document_causal" if causal else "document", "q_doc": ids, "kv_doc": ids}
    scale = 0.4
    out, lse = oracle.attention_rows(q, k, v, mask, {"kind": "identity"}, scale)
    out, lse = out.reshape(H, L, D), lse.reshape(H, L)
    start = 0
    for n in lens:
        sl = slice(start, start + n)
        tq, tk, tv = (torch.from_numpy(x[0, :, sl]).double() for x in (q, k, v))
        ro, rl = _sdpa_out_lse(tq, tk, tv, scale, causal)
        np.testing.assert_allclose(out[:, sl], ro.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, sl], rl.numpy(), rtol=0, atol=1e-12)
        start += n


def _torch_doc_mask(q_doc, kv_doc, causal):
    m = torch.from_numpy(q_doc)[:, None] == torch.from_numpy(kv_doc)[None, :]
    if causal:
        m &= torch.arange(len(q_doc))[:, None] >= torch.arange(len(kv_doc))[None, :]
    return m


@pytest.mark.parametrize("causal", [False, True])
def test_any_ids_match_sdpa_with_a_dense_mask(causal):
    """Unsorted ids and different query / key lengths; every query's document
    has a key at or before it, so SDPA is defined on every row."""
    q_doc = np.array([2, 0, 1, 1, 0, 2, 3, 1], np.int32)
    kv_doc = np.array([0, 2, 1, 3, 0, 1, 2, 1, 0, 3, 2], np.int32)
    if causal:
        # make every row see a key at or before it: key i has q_doc[i]'s id
        kv_doc[:len(q_doc)] = q_doc
    Lq, Lk, D, H = len(q_doc), len(kv_doc), 8, 3
    q, k, v = _rand((1, H, Lq, D), 4), _rand((1, H, Lk, D), 5), _rand((1, H, Lk, D), 6)
    mask = {"kind": "document_causal" if causal else "document", "q_doc": q_doc, "kv_doc": kv_doc}
    out, _ = oracle.attention_rows(q, k, v, mask, {"kind": "identity"}, 0.3)
    tq, tk, tv = (torch.from_numpy(x).double() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=_torch_doc_mask(q_doc, kv_doc, causal), scale=0.3)
    np.testing.assert_allclose(out.reshape(1, H, Lq, D), ref.numpy(), rtol=0, atol=1e-12)


def test_backward_matches_sdpa_autograd():
    q_doc = np.array([0, 0, 0, 1, 1, 2, 2, 2, 2, 3], np.int32)
    Lq = Lk = len(q_doc)
    B, H, D = 2, 2, 8
    q, k, v = _rand((B, H, Lq, D), 7), _rand((B, H, Lk, D), 8), _rand((B, H, Lk, D), 9)
    dout = _rand((B, H, Lq, D), 10)
    for causal in (False, True):
        mask = {"kind": "document_causal" if causal else "document", "q_doc": q_doc,
                "kv_doc": q_doc}
        dq, dk, dv = oracle.attention_backward(q, k, v, dout, mask, {"kind": "identity"}, 0.5)
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=_torch_doc_mask(q_doc, q_doc, causal), scale=0.5)
        out.backward(torch.tensor(dout, dtype=torch.float64))
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_one_document_is_the_plain_mask(causal):
    L, D = 40, 8
    ids = np.full(L, 7, np.int32)
    q, k, v = _rand((1, 2, L, D), 11), _rand((1, 2, L, D), 12), _rand((1, 2, L, D), 13)
    a = oracle.attention_rows(q, k, v, {"kind": "document_causal" if causal else "document",
                                        "q_doc": ids, "kv_doc": ids}, {"kind": "identity"}, 0.2)
    b = oracle.attention_rows(q, k, v, {"kind": "causal" if causal else "noop"},
                              {"kind": "identity"}, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_block_arrays_hand_worked():
    with open(os.path.join(GOLDEN, "document_block_mask.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ids = np.array(c["ids"], np.int32)
        mask = {"kind": c["kind"], "q_doc": ids, "kv_doc": ids}
        L = len(ids)
        got = oracle.block_mask(mask, L, L, c["block"], c["block"])
        for name, g in zip(["kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                            "full_kv_indices"], got):
            assert g.tolist() == c[name], (c["kind"], name, g.tolist())
        assert oracle.count_visible(mask, L, L) == c["visible_pairs"]


def test_missing_or_short_ids_are_rejected():
    with pytest.raises(ValueError):
        oracle.count_visible({"kind": "document"}, 4, 4)
    with pytest.raises(ValueError):
        oracle.count_visible({"kind": "document", "q_doc": np.zeros(3, np.int32),
                              "kv_doc": np.zeros(4, np.int32)}, 4, 4)


def test_document_workload_pair_count_closed_form():
    """Packed causal documents of lengths n_d: sum_d n_d (n_d + 1) / 2 visible
    pairs (checked on the workload's id recipe at 4096 tokens)."""
    from block_sparse_masked_flexattention_amd.inputs import with_doc_ids, workload
    cfg = workload("document_causal", q_len=4096, kv_len=4096)
    mask = with_doc_ids(cfg)
    _, counts = np.unique(mask["q_doc"].numpy(), return_counts=True)
    assert counts.sum() == 4096 and len(counts) > 2
    want = int((counts * (counts + 1) // 2).sum())
    assert oracle.count_visible(mask, 4096, 4096) == want
    assert oracle.count_visible(dict(mask, kind="document"), 4096, 4096) == int((counts ** 2).sum())
