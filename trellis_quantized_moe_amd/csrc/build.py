"""Build libexl3moe.so (gfx950) in-tree with hipcc.

Usage: python -m trellis_quantized_moe_amd.csrc.build  (or call build()).
Every call recompiles all sources. Objects go to csrc/_build/, the library to
trellis_quantized_moe_amd/libexl3moe.so. The build fails if any kernel uses
scratch memory (see check_no_scratch); the compiler's per-kernel register,
LDS and occupancy figures are written to csrc/_build/kernel_resources.txt.
"""

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libexl3moe.so")
SOURCES = ["gemm.hip", "gemm_wide.hip", "rotate.hip", "combine.hip", "route_pack.hip", "host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 instructions stay off (see the build notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


_RES = re.compile(r"remark: +(Function Name|ScratchSize \[bytes/lane\]|VGPRs|AGPRs|"
                  r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)")


def kernel_resources(stderr):
    """Per-kernel resource figures from hipcc's kernel-resource-usage remarks:
    {mangled name: {"ScratchSize": .., "VGPRs": .., ...}}."""
    out, cur = {}, None
    for m in _RES.finditer(stderr):
        key, val = m.group(1).split(" [")[0], m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val)
    return out


def _compile(src):
    obj = os.path.join(HERE, "_build", os.path.splitext(src)[0] + ".o")
    cmd = ([HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
                              os.path.join(HERE, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj, kernel_resources(r.stderr)


def check_no_scratch(resources):
    """The GEMM kernels wait for their own loads with exact vmcnt counts
    written in inline asm; a register spill would add scratch loads and
    stores that those counts do not know about. No kernel of the library may
    use scratch, so a build where the compiler spills anywhere fails here."""
    bad = {k: v.get("ScratchSize") for k, v in resources.items() if v.get("ScratchSize", 0)}
    if bad:
        raise RuntimeError("kernels use scratch (register spills): %s" % bad)


def build(verbose=False):
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    resources = {}
    for _, res in done:
        resources.update(res)
    check_no_scratch(resources)
    with open(os.path.join(HERE, "_build", "kernel_resources.txt"), "w") as f:
        for name in sorted(resources):
            f.write("%s %s\n" % (name, " ".join("%s=%s" % kv for kv in sorted(resources[name].items()))))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
