"""Compile libflexattn.so for gfx950 with hipcc (no GPU needed).

    python -m block_sparse_masked_flexattention_amd.build [-j N]

Each .hip source is compiled to an object in parallel, then linked into
``block_sparse_masked_flexattention_amd/libflexattn.so`` next to this file.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libflexattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# amdgpu-mfma-vgpr-form: keep matrix-instruction accumulators in ordinary
# VGPRs; the softmax reads every score and rescales the output accumulator,
# and accumulators parked in AGPRs would cost a copy each way.
# -fno-honor-nans, device pass only: lets fmaxf become a bare v_max/v_max3
# (no NaN-quieting copy of each operand); inputs holding NaN give
# unspecified outputs.  Infinities are still honoured (masked scores are
# -inf).  The host pass honours NaNs: its argument checks test for them.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Xarch_device", "-fno-honor-nans",
    "-munsafe-fp-atomics", "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stdout))
    if r.stdout.strip():
        # the host pass does not know the gfx feature flag; show anything else
        lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(jobs: int | None = None, extra=(), out: str | None = None,
          build_dir: str | None = None) -> str:
    """Compile every .hip source and link the library.  `extra` adds hipcc
    flags; `out` / `build_dir` place a variant build elsewhere."""
    out = out or LIB_PATH
    build_dir = build_dir or BUILD_DIR
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra), build_dir), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    args = ap.parse_args(argv)
    print(build(args.j))


if __name__ == "__main__":
    main()
