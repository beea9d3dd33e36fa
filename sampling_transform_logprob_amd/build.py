"""Build ``libstce.so`` (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libstce.so")
SOURCES = ["kernels.hip", "select.hip", "sparse.hip", "api.hip"]

FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 arithmetic stays off: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # per-kernel register, LDS and scratch figures (checked below)
    "-Rpass-analysis=kernel-resource-usage",
]


def scratch_kernels(remarks: str) -> list:
    """(kernel, bytes per lane) of every kernel the compiler gave private
    scratch memory (register spills or private arrays): in the products such
    memory costs an order of magnitude of their time, and the entry point
    that allocates nothing must not need it."""
    import re
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libstce.so")
    bad = scratch_kernels(res.stderr)
    if bad:
        os.remove(LIB + ".tmp")
        raise RuntimeError("kernels with private scratch memory: " + ", ".join(f"{n} ({b} B/lane)" for n, b in bad))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
