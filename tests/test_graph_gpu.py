"""The library under HIP graph capture: the block-mask build and the forward
(and the backward) enqueue only kernels (no allocation, memset or
synchronisation inside a call), so a caller can capture them into a graph.
The graph is replayed several times, with eager work and synchronisations
between the replays, and every replay must equal the eager result bitwise."""
import numpy as np
import pytest
import torch

from block_sparse_masked_flexattention_amd import flexattn as fa
from block_sparse_masked_flexattention_amd.inputs import make_grad_inputs, make_inputs, workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _capture(fn):
    """Warm up on a side stream, capture fn, return the graph."""
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,over", [
    ("prefix_causal", dict(B=1, H=4, q_len=1000, kv_len=1000, mask={"kind": "prefix_causal", "prefix": 300})),
    ("sliding_window", dict(B=1, H=2, q_len=1500, kv_len=1500)),
    ("causal_rel_bias", dict(B=1, H=4, q_len=777, kv_len=777)),
])
def test_forward_graph_replays_match_eager(name, over):
    cfg = workload(name, **over)
    q, k, v = (t.to(DEV) for t in make_inputs(cfg))
    B, H, Lq, D = q.shape
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    out = torch.empty((B, H, Lq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=DEV)

    def step():
        fa.build_block_mask(*args, out=bm)
        fa.fwd(q, k, v, bm, cfg["score"], cfg["scale"], out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = _capture(step)
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        for a in bm.arrays():
            a.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "replay %d: out differs" % i
        assert torch.equal(lse, ref_lse), "replay %d: lse differs" % i
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)


def test_backward_graph_replays_match_eager():
    cfg = workload("prefix_causal", B=1, H=2, q_len=600, kv_len=600,
                   mask={"kind": "prefix_causal", "prefix": 200})
    q, k, v = (t.to(DEV) for t in make_inputs(cfg))
    dout = make_grad_inputs(cfg)[0].to(DEV)
    B, H, Lq, D = q.shape
    args = (cfg["mask"], cfg["q_len"], cfg["kv_len"], cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*args, device=DEV)
    bmt = fa.build_block_mask_t(*args, device=DEV)
    out, lse = fa.fwd(q, k, v, bm, cfg["score"], cfg["scale"], return_lse=True)
    grads = [torch.empty_like(q, dtype=torch.float32) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_floats(B, H, Lq), dtype=torch.float32, device=DEV)

    def step():
        fa.build_block_mask_t(*args, out=bmt)
        fa.bwd(q, k, v, out, dout, lse, bm, bmt, cfg["score"], cfg["scale"], workspace=ws,
               dq=grads[0], dk=grads[1], dv=grads[2])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in grads]
    g = _capture(step)
    for i in range(3):
        for t in grads:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("dq", "dk", "dv"), grads, ref):
            assert torch.equal(t, r), "replay %d: %s differs" % (i, name)
        step()
        torch.cuda.synchronize()
