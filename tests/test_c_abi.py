"""The C ABI from plain C: tests/c/abi_host.c and tests/c/abi_fuzz.c are compiled
with gcc against include/moonep.h only, linked to libmoonep.so and run (host-side
calls only: shape validation against the header's rules, workspace sizing, status
text and argument errors, no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from redundant_expert_balancing_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("prog", ["abi_host", "abi_fuzz"])
def test_plain_c_program_uses_the_abi(tmp_path, prog):
    L.lib()   # the library must be built
    libdir = os.path.dirname(L.LIB_PATH)
    exe = tmp_path / prog
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", f"{prog}.c"), "-L", libdir, "-lmoonep",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert f"{prog}: all checks passed" in res.stdout
