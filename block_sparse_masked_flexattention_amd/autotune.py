"""Block-size autotuning for the forward.

The pages' kernel is compiled from a template with a fixed Q_BLOCK x
KV_BLOCK tile; this library ships several tile shapes per head dim, and
which one is fastest depends on the mask (how many tiles are partial, how
long the tile lists are), the lengths and the head dims.  ``tune_fwd`` times
the forward on the caller's own tensors for every shape the library has and
remembers the winner per problem signature, so later calls with the same
signature get the answer without timing anything.

This is host logic around the library (block-mask builds and forward
launches through the C ABI, timed with HIP events); it adds no arithmetic of
its own.  It synchronises the stream and allocates block arrays, so it
belongs outside a captured or latency-critical region: tune once, then call
``flexattn.fwd`` with the chosen block mask.
"""
from __future__ import annotations

import threading
from dataclasses import dataclass, field

import torch

from . import flexattn as fa

# (q_block, kv_block) shapes built for every dtype / head-dim instance
TILE_SHAPES = ((64, 64), (128, 64), (128, 128))

_cache: dict = {}
_cache_lock = threading.Lock()


@dataclass
class TuneResult:
    q_block: int
    kv_block: int
    ms: dict = field(default_factory=dict)  # (q_block, kv_block) -> mean forward ms
    cached: bool = False


def signature(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: dict,
              score: dict | None, fwd_kw: dict) -> tuple:
    """What the choice may depend on: shapes, dtype, mask kind and
    parameters (document ids by content), score kind, forward options."""
    m = []
    for key in sorted(mask):
        val = mask[key]
        if isinstance(val, torch.Tensor):
            val = ("ids", int(val.numel()), hash(val.cpu().numpy().tobytes()))
        m.append((key, val))
    sc = tuple(sorted((score or {"kind": "identity"}).items()))
    opts = tuple(sorted((k_, bool(v_)) for k_, v_ in fwd_kw.items()
                        if k_ in ("use_subtiling", "prescale_qk", "return_lse", "return_max")))
    return (tuple(q.shape), int(k.shape[2]), int(v.shape[3]), str(q.dtype), tuple(m), sc, opts)


def candidates(q: torch.Tensor, v: torch.Tensor):
    """Tile shapes the library has for these head dims and dtype (sequence
    lengths of any size work with every shape: the last blocks may be
    ragged)."""
    D, Dv = int(q.shape[3]), int(v.shape[3])
    if D not in (64, 128) or Dv not in (64, 128):
        return []
    return list(TILE_SHAPES)


def tune_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: dict,
             score: dict | None = None, scale: float | None = None, *, reps: int = 10,
             warmup: int = 3, use_cache: bool = True, **fwd_kw) -> TuneResult:
    """Time the forward for every candidate tile shape on these tensors and
    return the fastest (ties go to the earlier shape).  ``fwd_kw`` are
    passed to ``flexattn.fwd`` (e.g. use_subtiling, return_lse)."""
    key = signature(q, k, v, mask, score, fwd_kw)
    if use_cache:
        with _cache_lock:
            hit = _cache.get(key)
        if hit is not None:
            return TuneResult(hit.q_block, hit.kv_block, dict(hit.ms), cached=True)
    cands = candidates(q, v)
    if not cands:
        raise ValueError("no built forward instance for head dims %d / %d and %s"
                         % (q.shape[3], v.shape[3], q.dtype))
    Lq, Lk = int(q.shape[2]), int(k.shape[2])
    stream = torch.cuda.current_stream(q.device)
    ms = {}
    for qb, kb in cands:
        bm = fa.build_block_mask(mask, Lq, Lk, qb, kb, device=q.device)
        for _ in range(warmup):
            fa.fwd(q, k, v, bm, score, scale, **fwd_kw)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fa.fwd(q, k, v, bm, score, scale, **fwd_kw)
            b.record(stream)
        torch.cuda.synchronize(q.device)
        ms[(qb, kb)] = sum(a.elapsed_time(b) for a, b in evs) / reps
    best = min(cands, key=lambda c: (ms[c], cands.index(c)))
    res = TuneResult(best[0], best[1], ms)
    if use_cache:
        with _cache_lock:
            _cache[key] = res
    return res


def clear_cache():
    with _cache_lock:
        _cache.clear()
