"""Build libtail.so (the decode-tail HIP library) in-tree for gfx950.

    python -m decode_sampling_tail_amd.build [--asm DIR]

Every .hip source under csrc/ is compiled by hipcc into one shared library
next to this file.  `--asm DIR` also keeps the AMD assembly of the device
code in DIR (for register / instruction inspection).
"""
from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libtail.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    # packed fp32 VALU forms stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the decode-tail library)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, f"-I{INCLUDE}", "-o", tmp, *sources()]
    cwd = None
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd.insert(1, "-save-temps")
        cwd = asm_dir
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libtail.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None)
    a = ap.parse_args()
    print(build(a.asm, verbose=True))
