"""CPU-only checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments on the host (no call here reaches a
kernel launch)."""
import ctypes
import os
import re

import pytest

from block_sparse_masked_flexattention_amd import flexattn as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "flexattn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(flex_attn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.flex_attn_abi_version() == fa.ABI_VERSION


def test_strerror():
    for code in (0, 1, 2, 3, 99, -1):
        assert isinstance(fa.strerror(code), str) and fa.strerror(code)
    assert fa.strerror(0) == "success"


@pytest.mark.parametrize("q_len,kv_len,qb,kb,expect", [
    (4096, 4096, 128, 64, (32, 64)),
    (1000, 1000, 128, 64, (8, 16)),
    (0, 5, 64, 64, (0, 1)),
    (1, 0, 64, 64, (1, 0)),
    (129, 257, 128, 128, (2, 3)),
])
def test_block_mask_dims(q_len, kv_len, qb, kb, expect):
    assert fa.block_mask_dims(q_len, kv_len, qb, kb) == expect


@pytest.mark.parametrize("args", [(-1, 4, 64, 64), (4, -1, 64, 64), (4, 4, 0, 64), (4, 4, 64, -2)])
def test_block_mask_dims_rejects(args):
    with pytest.raises(fa.FlexAttnError) as e:
        fa.block_mask_dims(*args)
    assert e.value.code == fa.FLEX_E_INVALID_ARG


def _build(mask, q_len=128, kv_len=128, qb=64, kb=64, ptr=0x1000, bounds=None, t=False):
    md = fa.mask_desc(mask) if isinstance(mask, dict) else mask
    fn = fa.load().flex_attn_build_block_mask_t if t else fa.load().flex_attn_build_block_mask
    return fn(ctypes.byref(md) if md is not None else None, q_len, kv_len, qb, kb,
              ptr, ptr, ptr, ptr, bounds, None)


def test_build_block_mask_rejects_on_host():
    assert _build(None) == fa.FLEX_E_INVALID_ARG
    assert _build({"kind": "causal"}, q_len=-1) == fa.FLEX_E_INVALID_ARG
    assert _build({"kind": "causal"}, qb=0) == fa.FLEX_E_INVALID_ARG
    assert _build({"kind": "causal"}, kb=2048) == fa.FLEX_E_INVALID_ARG
    assert _build({"kind": "sliding_window", "window": 3, "window_min": 5}) == fa.FLEX_E_INVALID_ARG
    assert _build({"kind": "sliding_window", "window": 3, "window_min": -1}) == fa.FLEX_E_INVALID_ARG
    assert _build({"kind": "prefix_causal", "prefix": -3}) == fa.FLEX_E_INVALID_ARG
    assert _build(fa.MaskDesc(7, 0, 0, 0)) == fa.FLEX_E_UNSUPPORTED
    assert _build({"kind": "causal"}, ptr=None) == fa.FLEX_E_INVALID_ARG
    # document kinds need their id arrays and the bounds output
    for t in (False, True):
        assert _build(fa.MaskDesc(4, 0, 0, 0, None, 0x1000), bounds=0x1000, t=t) == fa.FLEX_E_INVALID_ARG
        assert _build(fa.MaskDesc(5, 0, 0, 0, 0x1000, None), bounds=0x1000, t=t) == fa.FLEX_E_INVALID_ARG
        assert _build(fa.MaskDesc(4, 0, 0, 0, 0x1000, 0x1000), bounds=None, t=t) == fa.FLEX_E_INVALID_ARG
    assert _build(fa.MaskDesc(6, 0, 0, 0)) == fa.FLEX_E_UNSUPPORTED
    # nothing to do: no launch, success
    assert _build({"kind": "causal"}, q_len=0, ptr=None) == fa.FLEX_OK
    assert _build(fa.MaskDesc(4, 0, 0, 0, None, None), q_len=0, kv_len=0, ptr=None) == fa.FLEX_OK


def _fwd(B=1, H=1, Lq=128, Lk=128, D=64, dtype=fa.DTYPE_BF16, qb=64, kb=64, mask=None,
         bm_lens=None, score=None, scale=0.125, out_dtype=fa.DTYPE_BF16, ptr=0x1000,
         nq=None, nk=None, lse=None, max_out=None, opt=None, Dv=None):
    mask = mask or {"kind": "causal"}
    nq_, nk_ = -(-Lq // qb), -(-Lk // kb)
    lq, lk = bm_lens or (Lq, Lk)
    bm = fa.BlockMaskStruct(fa.mask_desc(mask), lq, lk, qb, kb,
                            nq if nq is not None else nq_, nk if nk is not None else nk_,
                            ptr, ptr, ptr, ptr)
    sd = None if score is None else ctypes.byref(score)
    od = None if opt is None else ctypes.byref(opt)
    return fa.load().flex_attn_fwd(ptr, ptr, ptr, dtype, B, H, Lq, Lk, D, D if Dv is None else Dv,
                                   ctypes.byref(bm), sd,
                                   scale, ptr, out_dtype, lse, max_out, od, None)


def test_fwd_rejects_on_host():
    lib = fa.load()
    assert lib.flex_attn_fwd(0x1000, 0x1000, 0x1000, 0, 1, 1, 128, 128, 64, 64, None, None,
                             0.125, 0x1000, 0, None, None, None, None) == fa.FLEX_E_INVALID_ARG
    assert _fwd(B=-1) == fa.FLEX_E_INVALID_ARG
    assert _fwd(dtype=5) == fa.FLEX_E_INVALID_ARG
    assert _fwd(out_dtype=9) == fa.FLEX_E_INVALID_ARG
    assert _fwd(bm_lens=(64, 128)) == fa.FLEX_E_INVALID_ARG      # mask built for other lengths
    assert _fwd(nq=3) == fa.FLEX_E_INVALID_ARG                   # wrong block count
    assert _fwd(D=96) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(Dv=96) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(Dv=0) == fa.FLEX_E_INVALID_ARG
    assert _fwd(Dv=96, dtype=fa.DTYPE_FP32) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(qb=32, kb=32) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(scale=0.0) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(scale=float("nan")) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(mask={"kind": "sliding_window", "window": 1, "window_min": 2}) == fa.FLEX_E_INVALID_ARG
    assert _fwd(score=fa.ScoreDesc(1, 4, 8.0), H=8) == fa.FLEX_E_INVALID_ARG  # num_heads != H
    assert _fwd(score=fa.ScoreDesc(5, 1, 8.0)) == fa.FLEX_E_UNSUPPORTED
    assert _fwd(score=fa.ScoreDesc(1, 1, 8.0, 0x1002)) == fa.FLEX_E_INVALID_ARG  # slopes misaligned
    assert _fwd(score=fa.ScoreDesc(1, 1, float("nan"))) == fa.FLEX_E_INVALID_ARG  # no table: finite
    assert _fwd(score=fa.ScoreDesc(1, 4, 8.0, 0x1000), H=8) == fa.FLEX_E_INVALID_ARG
    assert _fwd(ptr=0x1008) == fa.FLEX_E_INVALID_ARG            # not 16-byte aligned
    assert _fwd(ptr=None) == fa.FLEX_E_INVALID_ARG
    assert _fwd(mask={"kind": "document"}) == fa.FLEX_E_INVALID_ARG  # no row bounds
    assert _fwd(lse=0x1002) == fa.FLEX_E_INVALID_ARG            # lse not 4-byte aligned
    assert _fwd(max_out=0x1001) == fa.FLEX_E_INVALID_ARG        # max not 4-byte aligned
    # PRESCALE_QK: scale * log2 e must stay a finite, non-zero float
    assert _fwd(scale=3e38, opt=fa.FwdOptions(0, 1, 0, 0)) == fa.FLEX_E_UNSUPPORTED
    # empty problems succeed without launching anything
    assert _fwd(B=0, ptr=None, nq=None) == fa.FLEX_OK
    assert _fwd(Lq=0, ptr=None) == fa.FLEX_OK


def _bwd(B=1, H=1, Lq=128, Lk=128, D=64, Dv=None, dtype=fa.DTYPE_BF16, qb=64, kb=64, mask=None,
         score=None, scale=0.125, grad_dtype=fa.DTYPE_FP32, ptr=0x1000, ws=0x1000,
         t_blocks=None, lse=0x1000):
    mask = mask or {"kind": "causal"}
    nq, nk = -(-Lq // qb), -(-Lk // kb)
    bm = fa.BlockMaskStruct(fa.mask_desc(mask), Lq, Lk, qb, kb, nq, nk, ptr, ptr, ptr, ptr)
    tq, tk = t_blocks or (qb, kb)
    bmt = fa.BlockMaskTStruct(tq, tk, nq, nk, ptr, ptr, ptr, ptr)
    sd = None if score is None else ctypes.byref(score)
    return fa.load().flex_attn_bwd(ptr, ptr, ptr, ptr, ptr, lse, None, dtype, B, H, Lq, Lk, D,
                                   D if Dv is None else Dv, ctypes.byref(bm), ctypes.byref(bmt), sd, scale,
                                   ptr, ptr, ptr, grad_dtype, ws, None)


def test_bwd_rejects_on_host():
    lib = fa.load()
    n = ctypes.c_int64()
    assert lib.flex_attn_bwd_workspace_floats(2, 3, 100, ctypes.byref(n)) == fa.FLEX_OK
    assert n.value == 2 * 2 * 3 * 100
    assert lib.flex_attn_bwd_workspace_floats(-1, 3, 100, ctypes.byref(n)) == fa.FLEX_E_INVALID_ARG
    assert _bwd(B=-1) == fa.FLEX_E_INVALID_ARG
    assert _bwd(dtype=7) == fa.FLEX_E_INVALID_ARG
    assert _bwd(grad_dtype=7) == fa.FLEX_E_INVALID_ARG
    assert _bwd(t_blocks=(128, 64)) == fa.FLEX_E_INVALID_ARG    # transposed mask of other blocks
    assert _bwd(D=96) == fa.FLEX_E_UNSUPPORTED                 # head dims 64 and 128 only
    assert _bwd(Dv=96) == fa.FLEX_E_UNSUPPORTED
    assert _bwd(Dv=0) == fa.FLEX_E_INVALID_ARG
    assert _bwd(dtype=fa.DTYPE_FP32, Dv=96) == fa.FLEX_E_UNSUPPORTED
    assert _bwd(dtype=fa.DTYPE_FP32, qb=32, kb=32) == fa.FLEX_E_UNSUPPORTED
    assert _bwd(qb=32, kb=32) == fa.FLEX_E_UNSUPPORTED
    assert _bwd(scale=0.0) == fa.FLEX_E_UNSUPPORTED
    assert _bwd(mask={"kind": "prefix_causal", "prefix": -1}) == fa.FLEX_E_INVALID_ARG
    assert _bwd(score=fa.ScoreDesc(1, 4, 8.0), H=8) == fa.FLEX_E_INVALID_ARG
    assert _bwd(score=fa.ScoreDesc(1, 1, 8.0, 0x1001)) == fa.FLEX_E_INVALID_ARG  # slopes misaligned
    assert _bwd(ptr=0x1008) == fa.FLEX_E_INVALID_ARG           # not 16-byte aligned
    assert _bwd(ws=None) == fa.FLEX_E_INVALID_ARG              # workspace required
    assert _bwd(lse=None) == fa.FLEX_E_INVALID_ARG             # lse required
    # empty problems succeed without launching anything
    assert _bwd(B=0, ptr=None, ws=None, lse=None) == fa.FLEX_OK


def test_struct_layouts_match_the_header(tmp_path):
    """Every ctypes structure of the binding has the size and field offsets
    the C compiler gives the header's struct (compiled here with gcc)."""
    import subprocess
    structs = {
        "flex_mask_desc": fa.MaskDesc,
        "flex_block_mask": fa.BlockMaskStruct,
        "flex_block_mask_t": fa.BlockMaskTStruct,
        "flex_score_desc": fa.ScoreDesc,
        "flex_fwd_options": fa.FwdOptions,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "flexattn.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append('  printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for fname, _ in cls._fields_:
            lines.append('  printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, fname, cname, fname))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        parts = line.split()
        if len(parts) == 3:
            got[(parts[0], parts[1])] = int(parts[2])
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)
