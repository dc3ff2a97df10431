"""Build libqwg.so in-tree with hipcc for gfx950 (hand-written HIP kernels + host runtime)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqwg.so")
SOURCES = ["qwg_gemv.hip", "qwg_ops.hip", "qwg_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed-fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _obj(src: str) -> str:
    return os.path.join(CSRC, "_build", os.path.splitext(src)[0] + ".o")


def build(verbose: bool = False, jobs: int = 3) -> str:
    """Compile every source and link libqwg.so. Always recompiles (this is the build check)."""
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)

    def compile_one(src):
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", _obj(src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return src

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + [_obj(s) for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
