"""Build libmqa_topk.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libmqa_topk.so")
SOURCES = ["fused.hip", "dense.hip", "probe.hip", "api.hip"]
HEADERS = ["common.h", "launch.h"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(out: str) -> list[str]:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-o", out] + \
           [os.path.join(CSRC, s) for s in SOURCES]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + \
           [os.path.join(ROOT, "include", "mqa_topk.h")]
    return any(os.path.getmtime(d) > t for d in deps)


def build(force: bool = True) -> str:
    """Compile the library (always when force, else only when missing/stale)."""
    if not force and not stale():
        return LIB
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    res = subprocess.run(command(tmp), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
