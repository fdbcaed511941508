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
# FLEXATTN_LIB: another build of the same library (for instance one with
# host-side sanitizers)
LIB_PATH = os.environ.get("FLEXATTN_LIB") or os.path.join(_HERE, "libflexattn.so")

FLEX_OK, FLEX_E_INVALID_ARG, FLEX_E_UNSUPPORTED, FLEX_E_HIP, FLEX_E_SCRATCH_LIMIT = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_FLOATS = 1 << 23
DTYPE_BF16, DTYPE_FP32 = 0, 1
MASK_KINDS = {"noop": 0, "causal": 1, "sliding_window": 2, "prefix_causal": 3,
              "document": 4, "document_causal": 5}
SCORE_KINDS = {"identity": 0, "rel_bias": 1}
ABI_VERSION = 8

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
    "flex_attn_bwd_noalloc",
    "flex_attn_mfma_peak_probe",
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
                ("bias_max", ctypes.c_float), ("slopes", ctypes.c_void_p)]


def score_desc(sc: dict | None, H: int, dev) -> ScoreDesc:
    """The score dict as the ABI struct: {"kind": "identity"} or
    {"kind": "rel_bias", "bias_max": 8.0} or {"kind": "rel_bias", "slopes": t}
    with t a float32 [H] tensor on the call's device (a per-head slope table,
    read by the kernels)."""
    sc = sc or {"kind": "identity"}
    slopes = sc.get("slopes")
    ptr = None
    if slopes is not None:
        _on_device(slopes, dev, "slopes", torch.float32, (H,))
        ptr = slopes.data_ptr()
    return ScoreDesc(SCORE_KINDS[sc["kind"]], int(sc.get("num_heads", H)),
                     float(sc.get("bias_max", 8.0)), ptr)


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
        lib.flex_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                              i32, i32, i32, ctypes.POINTER(BlockMaskStruct),
                                              ctypes.POINTER(BlockMaskTStruct),
                                              ctypes.POINTER(ScoreDesc), ctypes.c_float, vp, vp,
                                              vp, i32, vp]
        lib.flex_attn_bwd_noalloc.restype = i32
        lib.flex_attn_mfma_peak_probe.argtypes = [i32, i32, vp, vp, vp]
        lib.flex_attn_mfma_peak_probe.restype = i32
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


def _on_device(t, dev: torch.device, name: str, dtype=None, shape=None):
    """Raise ValueError unless t is a contiguous GPU tensor on `dev` (of
    `dtype` and `shape` when given): every pointer this binding passes to
    the library must be device memory the kernels can reach."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if t.device.type != "cuda" or t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _check_block_mask(bm, dev: torch.device, q_len: int, kv_len: int):
    """The block mask's arrays: int32, contiguous, on `dev`, sized for its
    block counts, and built for these sequence lengths."""
    if bm.q_len != q_len or bm.kv_len != kv_len:
        raise ValueError("block mask built for lengths (%d, %d), call has (%d, %d)"
                         % (bm.q_len, bm.kv_len, q_len, kv_len))
    nq, nk = block_mask_dims(q_len, kv_len, bm.q_block, bm.kv_block)
    for a, nm, shp in zip(bm.arrays(), ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                                        "full_kv_indices"), [(nq,), (nq, nk), (nq,), (nq, nk)]):
        _on_device(a, dev, nm, torch.int32, shp)
    if is_document(bm.mask):
        if bm.row_bounds is None:
            raise ValueError("a document mask needs row_bounds")
        _on_device(bm.row_bounds, dev, "row_bounds", torch.int32, (2 * q_len,))


def _check_block_mask_t(bmt, dev: torch.device, q_len: int, kv_len: int):
    if bmt.q_len != q_len or bmt.kv_len != kv_len:
        raise ValueError("transposed block mask built for other lengths")
    nq, nk = block_mask_dims(q_len, kv_len, bmt.q_block, bmt.kv_block)
    for a, nm, shp in zip(bmt.arrays(), ("q_num_blocks", "q_indices", "full_q_num_blocks",
                                         "full_q_indices"), [(nk,), (nk, nq), (nk,), (nk, nq)]):
        _on_device(a, dev, nm, torch.int32, shp)
    if is_document(bmt.mask):
        if bmt.col_bounds is None:
            raise ValueError("a document mask needs col_bounds")
        _on_device(bmt.col_bounds, dev, "col_bounds", torch.int32, (2 * kv_len,))


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
        if dev.type != "cuda":
            raise ValueError("the block mask is built on the GPU: device must be a cuda device")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        z = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
        out = BlockMask(dict(mask), q_len, kv_len, q_block, kv_block,
                        z(nq), z(nq, nk), z(nq), z(nq, nk),
                        z(2 * q_len) if is_document(mask) else None)
    elif (out.q_len, out.kv_len, out.q_block, out.kv_block) != (q_len, kv_len, q_block, kv_block):
        raise ValueError("out was made for other lengths or block sizes")
    arrs = out.arrays()
    dev = arrs[0].device
    if dev.type != "cuda":
        raise ValueError("block-mask arrays must be on a cuda device")
    for a, nm, shape in zip(arrs, ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                                   "full_kv_indices"), [(nq,), (nq, nk), (nq,), (nq, nk)]):
        _on_device(a, dev, nm, torch.int32, shape)
    if is_document(mask):
        if out.row_bounds is None:
            raise ValueError("a document mask needs row_bounds of 2 * q_len")
        _on_device(out.row_bounds, dev, "row_bounds", torch.int32, (2 * q_len,))
    for key in ("q_doc", "kv_doc"):
        if mask.get(key) is not None:
            _on_device(mask[key], dev, key, torch.int32)
    md = mask_desc(mask, q_len, kv_len)
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
    dev = q.device
    for t, nm in ((k, "k"), (v, "v")):
        _on_device(t, dev, nm)
    _check_block_mask(block_mask, dev, Lq, Lk)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, Lq, Dv), dtype=out_dtype, device=q.device)
    elif out.shape != (B, H, Lq, Dv) or out.dtype not in _DT or not out.is_contiguous():
        raise ValueError("bad out tensor")
    _on_device(out, dev, "out")
    if return_lse and lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _on_device(lse, dev, "lse", torch.float32, (B, H, Lq))
    if return_max and max_out is None:
        max_out = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if max_out is not None:
        _on_device(max_out, dev, "max_out", torch.float32, (B, H, Lq))
    sd = score_desc(score, H, dev)
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
        if dev.type != "cuda":
            raise ValueError("the block mask is built on the GPU: device must be a cuda device")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        z = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
        out = BlockMaskT(dict(mask), q_len, kv_len, q_block, kv_block,
                         z(nk), z(nk, nq), z(nk), z(nk, nq),
                         z(2 * kv_len) if is_document(mask) else None)
    elif (out.q_len, out.kv_len, out.q_block, out.kv_block) != (q_len, kv_len, q_block, kv_block):
        raise ValueError("out was made for other lengths or block sizes")
    arrs = out.arrays()
    dev = arrs[0].device
    if dev.type != "cuda":
        raise ValueError("transposed block-mask arrays must be on a cuda device")
    for a, nm, shape in zip(arrs, ("q_num_blocks", "q_indices", "full_q_num_blocks",
                                   "full_q_indices"), [(nk,), (nk, nq), (nk,), (nk, nq)]):
        _on_device(a, dev, nm, torch.int32, shape)
    if is_document(mask):
        if out.col_bounds is None:
            raise ValueError("a document mask needs col_bounds of 2 * kv_len")
        _on_device(out.col_bounds, dev, "col_bounds", torch.int32, (2 * kv_len,))
    for key in ("q_doc", "kv_doc"):
        if mask.get(key) is not None:
            _on_device(mask[key], dev, key, torch.int32)
    md = mask_desc(mask, q_len, kv_len)
    cb = out.col_bounds.data_ptr() if out.col_bounds is not None else None
    _check(load().flex_attn_build_block_mask_t(
        ctypes.byref(md), q_len, kv_len, q_block, kv_block,
        *[a.data_ptr() for a in arrs], cb, _stream_handle(dev)), "flex_attn_build_block_mask_t")
    return out


def mfma_peak_probe(n_workgroups: int, iters: int, device="cuda"):
    """Launch the matrix-unit peak microbenchmark once on the current stream
    (see flex_attn_mfma_peak_probe in include/flexattn.h).  Returns (FLOPs
    of the launch, sink tensor, clocks tensor); the caller times the launch
    and reads the clocks after synchronising."""
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError("the probe runs on a cuda device")
    sink = torch.empty(n_workgroups * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(n_workgroups * 4 * 2, dtype=torch.int64, device=dev)
    _check(load().flex_attn_mfma_peak_probe(n_workgroups, iters, sink.data_ptr(),
                                            clocks.data_ptr(), _stream_handle(sink.device)),
           "flex_attn_mfma_peak_probe")
    flops = float(n_workgroups) * 4 * iters * 4 * 32768
    return flops, sink, clocks


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
        dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
        write_dq: bool = True, noalloc: bool = False):
    """Gradients (dq, dk, dv) of the masked attention forward.  q/k/v/out/dout
    as in ``fwd`` (out and lse the forward's results), lse float32 [B,H,Lq].
    v, out, dout and dv may have a value head dim Dv other than q's D.
    ``write_dq=False`` (the WRITE_DQ kernel option) skips dq: the first
    result is then None.  ``noalloc=True`` calls flex_attn_bwd_noalloc,
    whose workspace is the library's own per-GPU scratch (no workspace
    argument; calls that overlap on one GPU race on it)."""
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
    dev = q.device
    for t, nm in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _on_device(t, dev, nm)
    _on_device(lse, dev, "lse", torch.float32, (B, H, Lq))
    if dlse is not None:
        _on_device(dlse, dev, "dlse", torch.float32, (B, H, Lq))
    _check_block_mask(block_mask, dev, Lq, Lk)
    _check_block_mask_t(block_mask_t, dev, Lq, Lk)
    gd = grad_dtype or torch.float32
    if gd not in _DT:
        raise ValueError("grad_dtype must be bfloat16 or float32")
    mk = lambda L, d: torch.empty((B, H, L, d), dtype=gd, device=q.device)
    if write_dq:
        dq = mk(Lq, D) if dq is None else dq
    elif dq is not None:
        raise ValueError("dq given with write_dq=False")
    dk = mk(Lk, D) if dk is None else dk
    dv = mk(Lk, Dv) if dv is None else dv
    for t, L, d in ((dq, Lq, D), (dk, Lk, D), (dv, Lk, Dv)):
        if t is None:
            continue
        if t.shape != (B, H, L, d) or t.dtype != gd or not t.is_contiguous():
            raise ValueError("bad gradient tensor")
        _on_device(t, dev, "gradient")
    nws = bwd_workspace_floats(B, H, Lq)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc=True takes no workspace")
    elif workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.float32, device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < nws:
        raise ValueError("workspace too small")
    else:
        _on_device(workspace, dev, "workspace", torch.float32)
    sd = score_desc(score, H, dev)
    bm = block_mask.as_struct()
    bmt = block_mask_t.as_struct()
    scale = default_scale(D) if scale is None else float(scale)
    common = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
              lse.data_ptr(), dlse.data_ptr() if dlse is not None else None, _DT[q.dtype],
              B, H, Lq, Lk, D, Dv, ctypes.byref(bm), ctypes.byref(bmt), ctypes.byref(sd), scale,
              dq.data_ptr() if dq is not None else None, dk.data_ptr(), dv.data_ptr(), _DT[gd])
    if noalloc:
        _check(load().flex_attn_bwd_noalloc(*common, _stream_handle(q.device)),
               "flex_attn_bwd_noalloc")
    else:
        _check(load().flex_attn_bwd(*common, workspace.data_ptr(), _stream_handle(q.device)),
               "flex_attn_bwd")
    return dq, dk, dv
