"""Build libloftq.so in-tree with hipcc for gfx950.

Every HIP/C++ source in csrc/ is compiled to an object of its own (in parallel,
under _build/) and the objects are linked into one shared library next to this
file.  Floating-point contraction is off (the codec's arithmetic is defined op
by op; the GEMMs call fmaf explicitly) and packed-fp32 instructions are disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libloftq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _filtered(stderr: str) -> str:
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    return "\n".join(ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln)


def _compile(src: str):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(HERE, "..", "include"), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, res


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    objs, failed = [], []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, res in ex.map(_compile, srcs):
            if res.returncode != 0:
                failed.append((src, res))
            else:
                objs.append(obj)
                if verbose and _filtered(res.stderr).strip():
                    sys.stderr.write(_filtered(res.stderr) + "\n")
    if failed:
        for src, res in failed:
            sys.stderr.write(f"--- {src}\n" + res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libloftq.so")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libloftq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
