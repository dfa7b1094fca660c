"""Build libmok.so (the HIP kernels and the C ABI) in place with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmok.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed fp32 arithmetic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source to an object in parallel, then link the shared library."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = [hipcc, *HIPCC_FLAGS, *lang, "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout)
    os.replace(tmp, LIB)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{text}")
    if verbose and text.strip():
        print(text)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
