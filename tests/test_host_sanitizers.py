"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host side only (each
-fsanitize= behind -Xarch_host; the device code is built as usual), and the
C-ABI validation cases of test_abi.py -- every rejected size, pointer, flag,
alignment and workspace, the workspace-size arithmetic -- run through it in
a subprocess with the sanitizer runtime preloaded.  Validation is pure host
logic that runs before any HIP call, so this needs no GPU.  Any report
(out-of-bounds access, integer overflow in the size arithmetic, ...) fails
the test.  The build is cached under _build/ by a hash of the sources."""
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_sampling_tail_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitizers")

FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
         "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
         "-Xarch_host", "-shared-libsan"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _asan_runtime(hipcc):
    out = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _build(hipcc):
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                     [os.path.join(ROOT, "include", "tail.h")])
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for p in sources:
        h.update(p.encode() + open(p, "rb").read())
    lib = os.path.join(OUT, f"libtail_sanitized_{h.hexdigest()[:12]}.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(OUT, exist_ok=True)
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [hipcc, *FLAGS, f"-I{os.path.join(ROOT, 'include')}", "-o", tmp,
           *sorted(glob.glob(os.path.join(CSRC, "*.hip")))]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    os.replace(tmp, lib)
    return lib


DRIVER = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import decode_sampling_tail_amd as dst
dst.LIB_PATH = {lib!r}
import test_abi
n = 0
for name in sorted(dir(test_abi)):
    if not name.startswith("test_"):
        continue
    fn = getattr(test_abi, name)
    if name == "test_topk_validation":
        for mirror in (False, True):
            fn(mirror)
    else:
        fn()
    n += 1
print("validation tests run:", n)
"""


def test_abi_validation_under_host_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    rt = _asan_runtime(hipcc)
    if rt is None:
        pytest.skip("the sanitizer runtime is not installed")
    lib = _build(hipcc)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm, "the host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = DRIVER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=600)
    report = res.stdout[-2000:] + res.stderr[-4000:]
    assert res.returncode == 0, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert "validation tests run:" in res.stdout, report
