"""The CPU ABI checks (test_abi_cpu.py) again, against a build of the C ABI
layer whose host code is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer: every argument check, layout computation and
error path of host.cpp runs under the sanitizers (no GPU is used). The
sanitized library is built from host.cpp plus the objects of the normal
build, and loaded in a fresh interpreter with the sanitizer runtime
preloaded; any report aborts that process."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_asan_and_ubsan():
    S = pytest.importorskip("trellis_quantized_moe_amd.csrc.build_sanitized")
    rt = S.runtime_path()
    if rt is None:
        pytest.skip("no sanitizer runtime in this toolchain")
    try:
        lib = S.build_sanitized()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = ("import sys\n"
            "from trellis_quantized_moe_amd import exl3\n"
            "exl3.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
            % (lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
