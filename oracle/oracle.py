"""Python side of the fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path never does, and this
module imports nothing from the product package.

``oracle.c`` holds the arithmetic (see its header for the passages each part
follows).  This wrapper only compiles it with gcc, marshals numpy arrays and
spreads independent query rows over host threads (each row is computed by the
same plain C loop; splitting rows changes no arithmetic).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
# FLEXATTN_ORACLE_LIB: another build of oracle.c (for instance one with
# sanitizers), loaded as it is
_LIB_ENV = os.environ.get("FLEXATTN_ORACLE_LIB")
_LIB_PATH = _LIB_ENV or os.path.join(_OUT_DIR, "liboracle.so")

MASK_KINDS = {"noop": 0, "causal": 1, "sliding_window": 2, "prefix_causal": 3,
              "document": 4, "document_causal": 5}
SCORE_KINDS = {"identity": 0, "rel_bias": 1}

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile oracle.c into a shared library with gcc; returns its path."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) and not _LIB_ENV:
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, i32p, f32p, f64p, i64p = (
            ctypes.c_int64,
            ctypes.POINTER(ctypes.c_int32),
            ctypes.POINTER(ctypes.c_float),
            ctypes.POINTER(ctypes.c_double),
            ctypes.POINTER(ctypes.c_int64),
        )
        # mask arguments: kind, window, window_min, prefix, q_doc, kv_doc
        m = [ctypes.c_int, i64, i64, i64, i32p, i32p]
        lib.oracle_mask_value.argtypes = m + [i64] * 4
        lib.oracle_mask_value.restype = ctypes.c_int
        lib.oracle_count_visible.argtypes = m + [i64] * 2
        lib.oracle_count_visible.restype = i64
        lib.oracle_block_mask.argtypes = m + [i64] * 4 + [i32p] * 4
        lib.oracle_block_mask.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = (
            [f32p, f32p, f32p] + [i64] * 6 + m
            + [ctypes.c_int, ctypes.c_double, f64p, ctypes.c_double, i64p, i64, f64p, f64p, f64p]
        )
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_block_mask_t.argtypes = m + [i64] * 4 + [i32p] * 4
        lib.oracle_block_mask_t.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = (
            [f32p, f32p, f32p, f32p, f32p] + [i64] * 6 + m
            + [ctypes.c_int, ctypes.c_double, f64p, ctypes.c_double, i64p, i64, f64p, f64p, f64p]
        )
        lib.oracle_attention_backward.restype = ctypes.c_int
        _lib = lib
        return lib


def _slopes(score: dict, H: int):
    """A per-head slope table (score["slopes"], H values, taken exactly as
    float64) or None for the formula."""
    t = score.get("slopes")
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(t, dtype=np.float64).reshape(-1))
    if a.shape != (H,):
        raise ValueError("slopes must hold one value per head")
    return a


def _doc_ptr(ids):
    """int32 pointer to a copy of a per-token document id array (the pointer
    keeps the copy alive), or None."""
    if ids is None:
        return None
    if hasattr(ids, "cpu"):
        ids = ids.cpu().numpy()
    a = np.ascontiguousarray(ids, dtype=np.int32)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _mask_args(mask: dict, q_len: int | None = None, kv_len: int | None = None):
    kind = MASK_KINDS[mask["kind"]]
    if kind >= 4:
        # the C code reads q_doc[i], kv_doc[j] for every i < q_len, j < kv_len
        for key, n in (("q_doc", q_len), ("kv_doc", kv_len)):
            if mask.get(key) is None:
                raise ValueError("document mask needs %s" % key)
            if n is not None and len(mask[key]) < n:
                raise ValueError("%s shorter than the sequence" % key)
    return (
        kind,
        int(mask.get("window", 0)),
        int(mask.get("window_min", 0)),
        int(mask.get("prefix", 0)),
        _doc_ptr(mask.get("q_doc")),
        _doc_ptr(mask.get("kv_doc")),
    )


def mask_value(mask: dict, i: int, j: int, q_len: int, kv_len: int) -> bool:
    r = _load().oracle_mask_value(*_mask_args(mask, q_len, kv_len), i, j, q_len, kv_len)
    if r < 0:
        raise ValueError("bad mask")
    return bool(r)


def count_visible(mask: dict, q_len: int, kv_len: int) -> int:
    return int(_load().oracle_count_visible(*_mask_args(mask, q_len, kv_len), q_len, kv_len))


def block_mask(mask: dict, q_len: int, kv_len: int, q_block: int, kv_block: int):
    """Brute-force block arrays: (kv_num_blocks, kv_indices, full_kv_num_blocks,
    full_kv_indices) as int32 numpy arrays of shapes [nQB], [nQB, nKVB]."""
    nq = -(-q_len // q_block)
    nk = -(-kv_len // kv_block)
    arrs = [
        np.zeros(nq, np.int32),
        np.zeros((nq, nk), np.int32),
        np.zeros(nq, np.int32),
        np.zeros((nq, nk), np.int32),
    ]
    ptrs = [a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) for a in arrs]
    r = _load().oracle_block_mask(
        *_mask_args(mask, q_len, kv_len), q_len, kv_len, q_block, kv_block, *ptrs
    )
    if r != 0:
        raise ValueError("oracle_block_mask rejected its arguments")
    return tuple(arrs)


def block_mask_t(mask: dict, q_len: int, kv_len: int, q_block: int, kv_block: int):
    """Brute-force transposed block arrays: (q_num_blocks, q_indices,
    full_q_num_blocks, full_q_indices) as int32 numpy arrays of shapes
    [nKVB], [nKVB, nQB]."""
    nq = -(-q_len // q_block)
    nk = -(-kv_len // kv_block)
    arrs = [
        np.zeros(nk, np.int32),
        np.zeros((nk, nq), np.int32),
        np.zeros(nk, np.int32),
        np.zeros((nk, nq), np.int32),
    ]
    ptrs = [a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) for a in arrs]
    r = _load().oracle_block_mask_t(
        *_mask_args(mask, q_len, kv_len), q_len, kv_len, q_block, kv_block, *ptrs
    )
    if r != 0:
        raise ValueError("oracle_block_mask_t rejected its arguments")
    return tuple(arrs)


def _cpu_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def attention_rows(q, k, v, mask: dict, score: dict, scale: float, rows=None,
                   threads: int | None = None, with_max: bool = False):
    """fp64 attention for selected rows.

    q: [B, H, Lq, D], k: [B, H, Lkv, D], v: [B, H, Lkv, Dv] float32 arrays (or
    anything numpy turns into float32 without changing values).  ``rows`` is an
    int64 array of flat row ids (b*H + h)*Lq + i; None means every row.
    Returns (out [n, Dv] float64, lse [n] float64), and with ``with_max`` also
    the row max of the visible scores [n] (-inf for a row with no key).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, H, Lq, D = q.shape
    Lkv, Dv = k.shape[2], v.shape[3]
    assert k.shape == (B, H, Lkv, D) and v.shape == (B, H, Lkv, Dv)
    if rows is None:
        rows = np.arange(B * H * Lq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    out = np.zeros((n, Dv), np.float64)
    lse = np.zeros(n, np.float64)
    mx = np.zeros(n, np.float64) if with_max else None
    score_kind = SCORE_KINDS[score.get("kind", "identity")]
    bias_max = float(score.get("bias_max", 8.0))
    slopes = _slopes(score, H)
    slp = slopes.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if slopes is not None else None
    lib = _load()
    margs = _mask_args(mask, Lq, Lkv)
    f32p = ctypes.POINTER(ctypes.c_float)
    qp, kp, vp = (a.ctypes.data_as(f32p) for a in (q, k, v))

    def run(lo, hi):
        if hi <= lo:
            return 0
        return lib.oracle_attention_rows(
            qp, kp, vp, B, H, Lq, Lkv, D, Dv, *margs, score_kind, bias_max, slp,
            float(scale),
            rows[lo:hi].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), hi - lo,
            out[lo:hi].ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            lse[lo:hi].ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            mx[lo:hi].ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if with_max else None,
        )

    nthr = threads or _cpu_threads()
    chunk = max(1, -(-n // (nthr * 4)))
    bounds = [(s, min(n, s + chunk)) for s in range(0, n, chunk)]
    if nthr == 1 or len(bounds) <= 1:
        codes = [run(lo, hi) for lo, hi in bounds]
    else:
        with ThreadPoolExecutor(nthr) as ex:
            codes = list(ex.map(lambda b: run(*b), bounds))
    if any(c != 0 for c in codes):
        raise ValueError("oracle_attention_rows rejected its arguments")
    return (out, lse, mx) if with_max else (out, lse)


def attention_backward(q, k, v, dout, mask: dict, score: dict, scale: float, dlse=None,
                       threads: int | None = None, heads=None):
    """fp64 gradients (dq, dk, dv) of every head, or of the flat heads
    b*H + h listed in ``heads`` (the others are left 0).

    q: [B, H, Lq, D], k: [B, H, Lkv, D], v: [B, H, Lkv, Dv], dout: [B, H, Lq, Dv]
    float32 arrays (exact values); dlse: [B, H, Lq] or None.  Heads are
    independent and are spread over host threads.
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    B, H, Lq, D = q.shape
    Lkv, Dv = k.shape[2], v.shape[3]
    assert k.shape == (B, H, Lkv, D) and v.shape == (B, H, Lkv, Dv)
    assert dout.shape == (B, H, Lq, Dv)
    if dlse is not None:
        dlse = np.ascontiguousarray(dlse, dtype=np.float32)
        assert dlse.shape == (B, H, Lq)
    dq = np.zeros((B, H, Lq, D), np.float64)
    dk = np.zeros((B, H, Lkv, D), np.float64)
    dv = np.zeros((B, H, Lkv, Dv), np.float64)
    score_kind = SCORE_KINDS[score.get("kind", "identity")]
    bias_max = float(score.get("bias_max", 8.0))
    slopes = _slopes(score, H)
    lib = _load()
    margs = _mask_args(mask, Lq, Lkv)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    slp = slopes.ctypes.data_as(f64p) if slopes is not None else None
    ptr = lambda a: a.ctypes.data_as(f32p)
    dlp = ptr(dlse) if dlse is not None else None
    heads = np.arange(B * H, dtype=np.int64) if heads is None else \
        np.ascontiguousarray(heads, dtype=np.int64)
    assert np.all((heads >= 0) & (heads < B * H))

    def run(t):
        hs = heads[t:t + 1]
        return lib.oracle_attention_backward(
            ptr(q), ptr(k), ptr(v), ptr(dout), dlp, B, H, Lq, Lkv, D, Dv, *margs,
            score_kind, bias_max, slp, float(scale),
            hs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1,
            dq.ctypes.data_as(f64p), dk.ctypes.data_as(f64p), dv.ctypes.data_as(f64p))

    nthr = threads or _cpu_threads()
    nh = len(heads)
    if nthr == 1 or nh <= 1:
        codes = [run(t) for t in range(nh)]
    else:
        with ThreadPoolExecutor(min(nthr, nh)) as ex:
            codes = list(ex.map(run, range(nh)))
    if any(c != 0 for c in codes):
        raise ValueError("oracle_attention_backward rejected its arguments")
    return dq, dk, dv


def threads_used(threads: int | None = None) -> int:
    return threads or _cpu_threads()
