"""Host logic of bench.py (no GPU): the visible-pair count behind the FLOP
metric, checked against closed forms and against the oracle's element mask
on small shapes, and the one-GPU guard."""
import subprocess
import sys
import os

import numpy as np
import pytest

import bench
from block_sparse_masked_flexattention_amd.inputs import WORKLOADS
from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# Visible (query, key) pairs per head of the five workloads, in closed form:
# causal L(L+1)/2; prefix P: L(L+1)/2 + P(P+1)/2 (the rows i <= P also see
# keys i+1..P); window W over length L: sum over rows of min(i, W) + 1.
def _window_pairs(L, W):
    return sum(min(i, W) + 1 for i in range(L))


@pytest.mark.parametrize("name,expect", [
    ("tiny_causal", 256 * 257 // 2),
    ("prefix_causal", 4096 * 4097 // 2 + 1025 * 1024 // 2),
    ("sliding_window", _window_pairs(8192, 256)),
    ("long_causal_d128", 16384 * 16385 // 2),
    ("causal_rel_bias", 32768 * 32769 // 2),
])
def test_visible_pairs_closed_forms(name, expect):
    cfg = WORKLOADS[name]
    assert bench.visible_pairs(cfg["mask"], cfg["q_len"], cfg["kv_len"]) == expect


def test_visible_pairs_printed_values():
    # the per-head counts quoted for the five workloads
    assert [bench.visible_pairs(WORKLOADS[n]["mask"], WORKLOADS[n]["q_len"], WORKLOADS[n]["kv_len"])
            for n in ("tiny_causal", "prefix_causal", "sliding_window", "long_causal_d128",
                      "causal_rel_bias")] == [32896, 8915456, 2072448, 134225920, 536887296]


@pytest.mark.parametrize("mask,lq,lk", [
    ({"kind": "causal"}, 37, 53),
    ({"kind": "causal"}, 70, 20),
    ({"kind": "sliding_window", "window": 9, "window_min": 2}, 40, 45),
    ({"kind": "prefix_causal", "prefix": 11}, 30, 25),
    ({"kind": "noop"}, 13, 17),
    ({"kind": "document_causal", "q_doc": np.array([0] * 5 + [1] * 9 + [2] * 6, np.int32),
      "kv_doc": np.array([0] * 5 + [1] * 9 + [2] * 6, np.int32)}, 20, 20),
])
def test_visible_pairs_match_the_oracle_mask(mask, lq, lk):
    dense = np.array([[oracle.mask_value(mask, i, j, lq, lk) for j in range(lk)] for i in range(lq)])
    assert bench.visible_pairs(mask, lq, lk) == int(dense.sum())


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
