"""ctypes binding of libflexattn.so (the C ABI in include/flexattn.h).

Argument marshalling only: every step of the attention forward and of the
block-mask build runs in the library's HIP kernels.  PyTorch supplies device
memory and the current HIP stream.  There is no fallback: if the library has
not been built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflexattn.so")

FLEX_OK, FLEX_E_INVALID_ARG, FLEX_E_UNSUPPORTED, FLEX_E_HIP = 0, 1, 2, 3
DTYPE_BF16, DTYPE_FP32 = 0, 1
MASK_KINDS = {"noop": 0, "causal": 1, "sliding_window": 2, "prefix_causal": 3,
              "document": 4, "document_causal": 5}
SCORE_KINDS = {"identity": 0, "rel_bias": 1}
ABI_VERSION = 5

# the functions include/flexattn.h declares
EXPORTED = (
    "flex_attn_abi_version",
    "flex_attn_strerror",
    "flex_attn_block_mask_dims",
    "flex_attn_build_block_mask",
    "flex_attn_build_block_mask_t",
    "flex_attn_fwd",
    "flex_attn_bwd_workspace_floats",
    "flex_attn_bwd",
)


class FlexAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, strerror(code), code))


class MaskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32),
                ("window_min", ctypes.c_int32), ("prefix", ctypes.c_int32),
                ("q_doc", ctypes.c_void_p), ("kv_doc", ctypes.c_void_p)]


class BlockMaskStruct(ctypes.Structure):
    _fields_ = [("mask", MaskDesc),
                ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
                ("n_q_blocks", ctypes.c_int32), ("n_kv_blocks", ctypes.c_int32),
                ("kv_num_blocks", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("full_kv_num_blocks", ctypes.c_void_p), ("full_kv_indices", ctypes.c_void_p),
                ("row_bounds", ctypes.c_void_p)]


class BlockMaskTStruct(ctypes.Structure):
    _fields_ = [("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
                ("n_q_blocks", ctypes.c_int32), ("n_kv_blocks", ctypes.c_int32),
                ("q_num_blocks", ctypes.c_void_p), ("q_indices", ctypes.c_void_p),
                ("full_q_num_blocks", ctypes.c_void_p), ("full_q_indices", ctypes.c_void_p),
                ("col_bounds", ctypes.c_void_p)]


class ScoreDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("bias_max", ctypes.c_float)]


class FwdOptions(ctypes.Structure):
    _fields_ = [("use_subtiling", ctypes.c_int32), ("prescale_qk", ctypes.c_int32),
                ("rows_guaranteed_safe", ctypes.c_int32),
                ("blocks_are_contiguous", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()


def load(path: str | None = None):
    """Load the built library (raises if it is missing: build it with
    ``python -m block_sparse_masked_flexattention_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise FileNotFoundError(
                "libflexattn.so is not built (%s); run "
                "`python -m block_sparse_masked_flexattention_amd.build`" % p)
        lib = ctypes.CDLL(p)
        i32, vp = ctypes.c_int32, ctypes.c_void_p
        lib.flex_attn_abi_version.argtypes = []
        lib.flex_attn_abi_version.restype = i32
        lib.flex_attn_strerror.argtypes = [i32]
        lib.flex_attn_strerror.restype = ctypes.c_char_p
        lib.flex_attn_block_mask_dims.argtypes = [i32, i32, i32, i32,
                                                  ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.flex_attn_block_mask_dims.restype = i32
        lib.flex_attn_build_block_mask.argtypes = [ctypes.POINTER(MaskDesc), i32, i32, i32, i32,
                                                   vp, vp, vp, vp, vp, vp]
        lib.flex_attn_build_block_mask.restype = i32
        lib.flex_attn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      ctypes.POINTER(BlockMaskStruct), ctypes.POINTER(ScoreDesc),
                                      ctypes.c_float, vp, i32, vp, vp,
                                      ctypes.POINTER(FwdOptions), vp]
        lib.flex_attn_fwd.restype = i32
        lib.flex_attn_build_block_mask_t.argtypes = [ctypes.POINTER(MaskDesc), i32, i32, i32,
                                                     i32, vp, vp, vp, vp, vp, vp]
        lib.flex_attn_build_block_mask_t.restype = i32
        lib.flex_attn_bwd_workspace_floats.argtypes = [i32, i32, i32,
                                                       ctypes.POINTER(ctypes.c_int64)]
        lib.flex_attn_bwd_workspace_floats.restype = i32
        lib.flex_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                      i32, ctypes.POINTER(BlockMaskStruct),
                                      ctypes.POINTER(BlockMaskTStruct),
                                      ctypes.POINTER(ScoreDesc), ctypes.c_float, vp, vp, vp,
                                      i32, vp, vp]
        lib.flex_attn_bwd.restype = i32
        if lib.flex_attn_abi_version() != ABI_VERSION:
            raise RuntimeError("libflexattn.so ABI version mismatch")
        if path is None:
            _lib = lib
        return lib


def strerror(code: int) -> str:
    return load().flex_attn_strerror(code).decode()


def _check(code: int, where: str):
    if code != FLEX_OK:
        raise FlexAttnError(code, where)


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) as float32 -- 0.125 at head_dim 64, 0.5 at 4."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))


def is_document(mask: dict) -> bool:
    return mask["kind"] in ("document", "document_causal")


def _doc_ptr(mask: dict, key: str, n: int | None):
    """Device pointer of a document id tensor (int32, contiguous, on the GPU,
    at least n long), or None."""
    t = mask.get(key)
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 \
            or not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError("%s must be a contiguous int32 GPU tensor" % key)
    if n is not None and t.numel() < n:
        raise ValueError("%s is shorter than the sequence" % key)
    return t.data_ptr()


def mask_desc(mask: dict, q_len: int | None = None, kv_len: int | None = None) -> MaskDesc:
    """The C descriptor.  Document kinds carry their id tensors
    (``mask["q_doc"]``, ``mask["kv_doc"]``: int32, non-decreasing)."""
    return MaskDesc(MASK_KINDS[mask["kind"]], int(mask.get("window", 0)),
                    int(mask.get("window_min", 0)), int(mask.get("prefix", 0)),
                    _doc_ptr(mask, "q_doc", q_len), _doc_ptr(mask, "kv_doc", kv_len))


def block_mask_dims(q_len: int, kv_len: int, q_block: int, kv_block: int):
    nq, nk = ctypes.c_int32(), ctypes.c_int32()
    _check(load().flex_attn_block_mask_dims(q_len, kv_len, q_block, kv_block,
                                            ctypes.byref(nq), ctypes.byref(nk)),
           "flex_attn_block_mask_dims")
    return nq.value, nk.value


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class BlockMask:
    """The kv half of a FlexAttention block mask, on the device."""
    mask: dict
    q_len: int
    kv_len: int
    q_block: int
    kv_block: int
    kv_num_blocks: torch.Tensor       # int32 [nQB]
    kv_indices: torch.Tensor          # int32 [nQB, nKVB]
    full_kv_num_blocks: torch.Tensor  # int32 [nQB]
    full_kv_indices: torch.Tensor     # int32 [nQB, nKVB]
    row_bounds: torch.Tensor | None = None  # document kinds: int32 [2 * q_len]

    def as_struct(self) -> BlockMaskStruct:
        nq, nk = self.kv_indices.shape
        return BlockMaskStruct(
            mask_desc(self.mask), self.q_len, self.kv_len, self.q_block, self.kv_block,
            nq, nk, self.kv_num_blocks.data_ptr(), self.kv_indices.data_ptr(),
            self.full_kv_num_blocks.data_ptr(), self.full_kv_indices.data_ptr(),
            self.row_bounds.data_ptr() if self.row_bounds is not None else None)

    def arrays(self):
        return (self.kv_num_blocks, self.kv_indices, self.full_kv_num_blocks,
                self.full_kv_indices)


def build_block_mask(mask: dict, q_len: int, kv_len: int, q_block: int, kv_block: int,
                     device="cuda", out: BlockMask | None = None) -> BlockMask:
    """Build the block arrays for a mask kind on the device (asynchronously,
    on the current stream).  ``out`` reuses existing arrays of the right size."""
    nq, nk = block_mask_dims(q_len, kv_len, q_block, kv_block)
    if out is None:
        dev = torch.device(device)
        z = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
        out = BlockMask(dict(mask), q_len, kv_len, q_block, kv_block,
                        z(nq), z(nq, nk), z(nq), z(nq, nk),
                        z(2 * q_len) if is_document(mask) else None)
    arrs = out.arrays()
    for a, shape in zip(arrs, [(nq,), (nq, nk), (nq,), (nq, nk)]):
        if a.dtype != torch.int32 or tuple(a.shape) != shape or not a.is_contiguous():
            raise ValueError("block-mask arrays have the wrong dtype/shape")
    if is_document(mask) and (out.row_bounds is None or out.row_bounds.numel() < 2 * q_len):
        raise ValueError("a document mask needs row_bounds of 2 * q_len")
    md = mask_desc(mask, q_len, kv_len)
    dev = arrs[0].device
    rb = out.row_bounds.data_ptr() if out.row_bounds is not None else None
    _check(load().flex_attn_build_block_mask(
        ctypes.byref(md), q_len, kv_len, q_block, kv_block,
        *[a.data_ptr() for a in arrs], rb, _stream_handle(dev)), "flex_attn_build_block_mask")
    return out


_DT = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_FP32}


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: BlockMask,
        score: dict | None = None, scale: float | None = None, *,
        out_dtype: torch.dtype | None = None, return_lse: bool = False,
        return_max: bool = False, use_subtiling: bool = False,
        prescale_qk: bool = False, rows_guaranteed_safe: bool = False,
        blocks_are_contiguous: bool = False, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, max_out: torch.Tensor | None = None):
    """Masked block-sparse attention forward.  q [B,H,Lq,D], k [B,H,Lkv,D],
    v [B,H,Lkv,Dv] (bfloat16 or float32, contiguous, on the GPU); out is
    [B,H,Lq,Dv].  Returns (out, lse) with lse
    None unless requested; with ``return_max`` (OUTPUT_MAX) returns
    (out, lse, max) where max is the float32 [B,H,Lq] row max of the scores.
    The remaining flags are the kernel options of the same names."""
    B, H, Lq, D = q.shape
    Lk, Dv = k.shape[2], v.shape[3]
    if k.shape != (B, H, Lk, D) or v.shape != (B, H, Lk, Dv):
        raise ValueError("q/k/v shapes disagree")
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q/k/v must share a dtype in {bfloat16, float32}")
    for t in (q, k, v):
        if not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("q/k/v must be contiguous GPU tensors")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, Lq, Dv), dtype=out_dtype, device=q.device)
    elif out.shape != (B, H, Lq, Dv) or out.dtype not in _DT or not out.is_contiguous():
        raise ValueError("bad out tensor")
    if return_lse and lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Lq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("bad lse tensor")
    if return_max and max_out is None:
        max_out = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if max_out is not None and (max_out.shape != (B, H, Lq) or max_out.dtype != torch.float32
                                or not max_out.is_contiguous()):
        raise ValueError("bad max_out tensor")
    sc = score or {"kind": "identity"}
    sd = ScoreDesc(SCORE_KINDS[sc["kind"]], int(sc.get("num_heads", H)),
                   float(sc.get("bias_max", 8.0)))
    opt = FwdOptions(int(bool(use_subtiling)), int(bool(prescale_qk)),
                     int(bool(rows_guaranteed_safe)), int(bool(blocks_are_contiguous)))
    bm = block_mask.as_struct()
    scale = default_scale(D) if scale is None else float(scale)
    _check(load().flex_attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype], B, H, Lq, Lk, D, Dv,
        ctypes.byref(bm), ctypes.byref(sd), scale, out.data_ptr(), _DT[out.dtype],
        lse.data_ptr() if lse is not None else None,
        max_out.data_ptr() if max_out is not None else None, ctypes.byref(opt),
        _stream_handle(q.device)), "flex_attn_fwd")
    lse_ret = lse if return_lse or lse is not None else None
    if return_max or max_out is not None:
        return out, lse_ret, max_out
    return out, lse_ret


@dataclass
class BlockMaskT:
    """The transposed block arrays (per kv-block column), on the device."""
    mask: dict
    q_len: int
    kv_len: int
    q_block: int
    kv_block: int
    q_num_blocks: torch.Tensor       # int32 [nKVB]
    q_indices: torch.Tensor          # int32 [nKVB, nQB]
    full_q_num_blocks: torch.Tensor  # int32 [nKVB]
    full_q_indices: torch.Tensor     # int32 [nKVB, nQB]
    col_bounds: torch.Tensor | None = None  # document kinds: int32 [2 * kv_len]

    def as_struct(self) -> BlockMaskTStruct:
        nk, nq = self.q_indices.shape
        return BlockMaskTStruct(self.q_block, self.kv_block, nq, nk,
                                self.q_num_blocks.data_ptr(), self.q_indices.data_ptr(),
                                self.full_q_num_blocks.data_ptr(),
                                self.full_q_indices.data_ptr(),
                                self.col_bounds.data_ptr() if self.col_bounds is not None else None)

    def arrays(self):
        return (self.q_num_blocks, self.q_indices, self.full_q_num_blocks,
                self.full_q_indices)


def build_block_mask_t(mask: dict, q_len: int, kv_len: int, q_block: int, kv_block: int,
                       device="cuda", out: BlockMaskT | None = None) -> BlockMaskT:
    """Build the transposed block arrays on the device (current stream)."""
    nq, nk = block_mask_dims(q_len, kv_len, q_block, kv_block)
    if out is None:
        dev = torch.device(device)
        z = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
        out = BlockMaskT(dict(mask), q_len, kv_len, q_block, kv_block,
                         z(nk), z(nk, nq), z(nk), z(nk, nq),
                         z(2 * kv_len) if is_document(mask) else None)
    arrs = out.arrays()
    for a, shape in zip(arrs, [(nk,), (nk, nq), (nk,), (nk, nq)]):
        if a.dtype != torch.int32 or tuple(a.shape) != shape or not a.is_contiguous():
            raise ValueError("transposed block-mask arrays have the wrong dtype/shape")
    if is_document(mask) and (out.col_bounds is None or out.col_bounds.numel() < 2 * kv_len):
        raise ValueError("a document mask needs col_bounds of 2 * kv_len")
    md = mask_desc(mask, q_len, kv_len)
    dev = arrs[0].device
    cb = out.col_bounds.data_ptr() if out.col_bounds is not None else None
    _check(load().flex_attn_build_block_mask_t(
        ctypes.byref(md), q_len, kv_len, q_block, kv_block,
        *[a.data_ptr() for a in arrs], cb, _stream_handle(dev)), "flex_attn_build_block_mask_t")
    return out


def bwd_workspace_floats(B: int, H: int, q_len: int) -> int:
    n = ctypes.c_int64()
    _check(load().flex_attn_bwd_workspace_floats(B, H, q_len, ctypes.byref(n)),
           "flex_attn_bwd_workspace_floats")
    return n.value


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
        dout: torch.Tensor, lse: torch.Tensor, block_mask: BlockMask,
        block_mask_t: BlockMaskT, score: dict | None = None, scale: float | None = None, *,
        dlse: torch.Tensor | None = None, grad_dtype: torch.dtype | None = None,
        workspace: torch.Tensor | None = None, dq: torch.Tensor | None = None,
        dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Gradients (dq, dk, dv) of the masked attention forward.  q/k/v/out/dout
    as in ``fwd`` (out and lse the forward's results), lse float32 [B,H,Lq].
    v, out, dout and dv may have a value head dim Dv other than q's D."""
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    Dv = v.shape[3] if v.dim() == 4 else -1
    if k.shape != (B, H, Lk, D) or v.shape != (B, H, Lk, Dv):
        raise ValueError("q/k/v shapes disagree")
    if out.shape != (B, H, Lq, Dv) or dout.shape != (B, H, Lq, Dv):
        raise ValueError("out/dout shapes disagree with q and v")
    if q.dtype not in _DT or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("q/k/v/out/dout must share a dtype in {bfloat16, float32}")
    for t in (q, k, v, out, dout):
        if not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("q/k/v/out/dout must be contiguous GPU tensors")
    if lse.shape != (B, H, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("bad lse tensor")
    if dlse is not None and (dlse.shape != (B, H, Lq) or dlse.dtype != torch.float32
                             or not dlse.is_contiguous()):
        raise ValueError("bad dlse tensor")
    gd = grad_dtype or torch.float32
    if gd not in _DT:
        raise ValueError("grad_dtype must be bfloat16 or float32")
    mk = lambda L, d: torch.empty((B, H, L, d), dtype=gd, device=q.device)
    dq = mk(Lq, D) if dq is None else dq
    dk = mk(Lk, D) if dk is None else dk
    dv = mk(Lk, Dv) if dv is None else dv
    for t, L, d in ((dq, Lq, D), (dk, Lk, D), (dv, Lk, Dv)):
        if t.shape != (B, H, L, d) or t.dtype != gd or not t.is_contiguous():
            raise ValueError("bad gradient tensor")
    nws = bwd_workspace_floats(B, H, Lq)
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.float32, device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < nws:
        raise ValueError("workspace too small")
    sc = score or {"kind": "identity"}
    sd = ScoreDesc(SCORE_KINDS[sc["kind"]], int(sc.get("num_heads", H)),
                   float(sc.get("bias_max", 8.0)))
    bm = block_mask.as_struct()
    bmt = block_mask_t.as_struct()
    scale = default_scale(D) if scale is None else float(scale)
    _check(load().flex_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dlse.data_ptr() if dlse is not None else None, _DT[q.dtype],
        B, H, Lq, Lk, D, Dv, ctypes.byref(bm), ctypes.byref(bmt), ctypes.byref(sd), scale,
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _DT[gd], workspace.data_ptr(),
        _stream_handle(q.device)), "flex_attn_bwd")
    return dq, dk, dv
