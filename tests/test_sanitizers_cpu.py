"""AddressSanitizer + UndefinedBehaviorSanitizer over the host code: the
oracle (built with gcc) and the C ABI's host-side validation (the library
built with the sanitizers on its host pass only; its device code is the
product's).  Each sanitized build runs the existing CPU tests in a child
process with the sanitizer runtime preloaded; any report aborts the child.

The sanitized builds are cached under tests/_san_build (not tracked), keyed
by a hash of their sources and flags: the first run compiles the library
once more (about a minute), later runs only run the tests."""
import hashlib
import os
import subprocess
import sys

import pytest

from block_sparse_masked_flexattention_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "tests", "_san_build")
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")

# host pass only: each -fsanitize= right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-g", "-O1"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(p.encode() + f.read())
    return h.hexdigest()


def _cached(name, paths, flags, make):
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, name)
    stamp = lib + ".sha256"
    want = _digest(paths, flags)
    if not (os.path.exists(lib) and os.path.exists(stamp) and open(stamp).read() == want):
        make(lib)
        with open(stamp, "w") as f:
            f.write(want)
    return lib


def _runtime(compiler, name):
    p = subprocess.run([compiler, "-print-file-name=" + name], stdout=subprocess.PIPE,
                       text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("%s has no %s" % (compiler, name))
    return p


def _run_child(tests, env_extra):
    env = dict(os.environ, **ENV_SAN, **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in tests]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-6000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stdout
    assert "runtime error:" not in r.stdout  # UBSan's report line


def test_oracle_under_asan_ubsan():
    def make(lib):
        subprocess.check_call(["gcc", *GCC_SAN, "-std=c99", "-fPIC", "-shared", "-o", lib,
                               ORACLE_SRC, "-lm"])
    lib = _cached("liboracle_san.so", [ORACLE_SRC], GCC_SAN, make)
    pre = " ".join(_runtime("gcc", n) for n in ("libasan.so", "libubsan.so"))
    _run_child(["test_oracle_pins.py", "test_oracle_document_pins.py",
                "test_oracle_options_pins.py", "test_oracle_backward_pins.py"],
               {"LD_PRELOAD": pre, "FLEXATTN_ORACLE_LIB": lib})


def test_abi_validation_under_asan_ubsan():
    srcs = libbuild.sources() + [os.path.join(ROOT, "include", "flexattn.h")]
    srcs += [os.path.join(libbuild.CSRC, f) for f in os.listdir(libbuild.CSRC)
             if f.endswith(".hpp")]

    def make(lib):
        libbuild.build(extra=HOST_SAN, out=lib, build_dir=os.path.join(OUT, "obj"))
    lib = _cached("libflexattn_san.so", srcs, libbuild.HIP_FLAGS + HOST_SAN, make)
    clang = os.path.join(os.path.dirname(libbuild.HIPCC), "..", "llvm", "bin", "clang")
    pre = _runtime(clang if os.path.exists(clang) else "clang", "libclang_rt.asan-x86_64.so")
    _run_child(["test_abi_cpu.py", "test_binding_cpu.py"],
               {"LD_PRELOAD": pre, "FLEXATTN_LIB": lib})
