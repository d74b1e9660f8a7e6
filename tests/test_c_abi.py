"""The C ABI from plain C (tests/c/abi_from_c.c): compiled with gcc against include/tmoe.h and linked
with the built libtmoe.so; host-only calls and fail-closed checks, so it runs without a GPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "trellis_quantized_moe_tmoe_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_abi_from_plain_c():
    assert os.path.exists(os.path.join(LIB_DIR, "libtmoe.so")), "build the library first"
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "abi_from_c")
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", LIB_DIR, "-ltmoe",
                        f"-Wl,-rpath,{LIB_DIR}", "-o", exe], check=True, capture_output=True, text=True)
        p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert p.returncode == 0, p.stdout + p.stderr
        assert p.stdout.strip().splitlines()[-1] == "PASSED"
