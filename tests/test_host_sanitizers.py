"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt into a temporary directory with both sanitizers on its host
code only (each flag behind -Xarch_host; the gfx950 code is compiled as usual), and
the two plain-C programs under tests/c are linked against it with ROCm's clang, whose
sanitizer runtime the library's instrumentation then uses. They exercise only host
paths: shape validation, workspace sizing, status text and every entry point's
argument checks (abi_host.c), and 200000 extreme and random shapes against the
header's stated rules (abi_fuzz.c). No GPU is needed or touched. Device code is not
sanitized: GPU AddressSanitizer needs xnack-enabled code objects, which this project
does not build."""
import os
import shutil
import subprocess

import pytest

from redundant_expert_balancing_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(
    not (os.path.exists(CLANG) and (shutil.which(HIPCC) or os.path.exists(HIPCC))),
    reason="ROCm clang / hipcc not available")


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitized")
    lib = d / "libmoonep.so"
    cmd = [HIPCC, *B.HIP_FLAGS, *HOST_SANITIZE, "-I", os.path.join(ROOT, "include"),
           *B.sources(), "-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-4000:]
    return d


@pytest.mark.parametrize("prog", ["abi_host", "abi_fuzz"])
def test_host_paths_clean_under_sanitizers(san_lib, prog):
    exe = san_lib / prog
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Werror",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", f"{prog}.c"),
                    "-L", str(san_lib), "-lmoonep", f"-Wl,-rpath,{san_lib}", "-o", str(exe)],
                   check=True, timeout=300)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert f"{prog}: all checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
