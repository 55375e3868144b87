"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
layer (host.cpp), for the CPU ABI tests.

host.cpp is recompiled with the sanitizers on its host code only (the
sanitizer flags are host-only; its device code and every other object are the
ones build() left in csrc/_build/) and linked into csrc/_build/libexl3moe_san.so.
Load it with the sanitizer runtime preloaded (runtime_path()).
"""

import glob
import os
import subprocess

from . import build as B

SAN_LIB = os.path.join(B.HERE, "_build", "libexl3moe_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan"]


def runtime_path():
    """The clang ASan shared runtime (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized():
    objs = [os.path.join(B.HERE, "_build", os.path.splitext(s)[0] + ".o")
            for s in B.SOURCES if s != "host.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError("run build() first: %s" % missing)
    host_o = os.path.join(B.HERE, "_build", "host_san.o")
    cmd = ([B.HIPCC] + B.FLAGS + HOST_SAN +
           ["-x", "hip", "-c", os.path.join(B.HERE, "host.cpp"), "-o", host_o])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    cmd = ([B.HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + HOST_SAN +
           ["-o", SAN_LIB] + objs + [host_o])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    return SAN_LIB
