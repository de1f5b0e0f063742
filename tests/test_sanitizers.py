"""Sanitizer builds, on the CPU: the oracle (gcc) and the host code of libdsa
(hipcc, host side only) built with AddressSanitizer and
UndefinedBehaviorSanitizer, then the oracle's pins and the C-ABI argument
checks run against those builds in a child process with the sanitizer
runtime preloaded (the Python interpreter itself is not instrumented).  A
planted out-of-bounds write shows that the instrumentation is live."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
ORACLE_SRC = os.path.join(ROOT, "oracle", "dsa_oracle.c")
CSRC = os.path.join(ROOT, "fp8_indexer_amd", "csrc")
from fp8_indexer_amd.build import SOURCES  # noqa: E402
ENV_BASE = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _gcc_runtime():
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True)
            .stdout.strip() for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc sanitizer runtimes not installed")
    return " ".join(libs)


def _build_oracle(out, src_text=None, tmp=None):
    src = ORACLE_SRC
    if src_text is not None:
        src = os.path.join(tmp, "oracle_mut.c")
        with open(src, "w") as f:
            f.write(src_text.replace('#include "dsa_oracle.h"',
                                     f'#include "{os.path.join(ROOT, "oracle", "dsa_oracle.h")}"'))
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fno-omit-frame-pointer", *san, "-o", out, src, "-lm"], check=True)


def _run_child(code, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV_BASE)
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=600, cwd=ROOT)


PINS = """
import sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import oracle_pins as P
with P.oracle_lib({lib!r}):
    for c in P.ALL_CHECKS:
        c()
print("PINS OK")
"""


def test_oracle_pins_under_asan_ubsan(tmp_path):
    pre = _gcc_runtime()
    lib = str(tmp_path / "liboracle_san.so")
    _build_oracle(lib)
    r = _run_child(PINS.format(tests=TESTS, root=ROOT, lib=lib), pre)
    assert r.returncode == 0 and "PINS OK" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_asan_catches_a_planted_overflow(tmp_path):
    """The same harness on an oracle whose top-k writes one slot past each
    output row must report a heap overflow (the last row's)."""
    pre = _gcc_runtime()
    src = open(ORACLE_SRC).read()
    anchor = "for (int32_t j = 0; j < K; ++j) o[j] = -1;"
    assert src.count(anchor) == 1
    lib = str(tmp_path / "liboracle_oob.so")
    _build_oracle(lib, src.replace(anchor, "for (int32_t j = 0; j <= K; ++j) o[j] = -1;"),
                  str(tmp_path))
    code = ("import sys, numpy as np\nsys.path.insert(0, %r)\nimport oracle\n"
            "L = oracle.lib(%r); oracle._lib = L\n"
            "print(oracle.topk(np.zeros((3, 10), np.float32), np.zeros(3, np.int32),"
            " np.full(3, 10, np.int32), 1, 3, 10, 4))\n") % (ROOT, lib)
    r = _run_child(code, pre)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("clang AddressSanitizer runtime not found")
    return hits[-1]


ABI = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import fp8_indexer_amd as dsa
dsa.LIB_PATH = {lib!r}
import test_abi as T
for name in ("test_version_and_status_strings", "test_indexer_rejects_bad_arguments",
             "test_topk_rejects_bad_arguments", "test_attention_rejects_bad_arguments",
             "test_prefill_rejects_null_and_inconsistent", "test_workspace_size_queries"):
    getattr(T, name)()
print("ABI OK")
"""


def test_host_code_under_asan_ubsan(tmp_path):
    """libdsa's host side (argument validation, workspace sizing, path
    choice) built with both sanitizers; the C-ABI rejection tests and size
    queries run against it (no kernel is launched: no GPU here)."""
    pre = _clang_asan_runtime()
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    objs = []
    procs = []
    for src in SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-c", os.path.join(CSRC, src), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out.decode()[-3000:]
    lib = str(tmp_path / "libdsa_san.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-o", lib, *objs], check=True, capture_output=True)
    r = _run_child(ABI.format(root=ROOT, tests=TESTS, lib=lib), pre)
    assert r.returncode == 0 and "ABI OK" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr
