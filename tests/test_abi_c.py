"""The C ABI used from plain C99: tests/c/abi_from_c.c is compiled with gcc
against include/vsa.h alone, linked to libvsa.so and run (host helpers and
argument checks only, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

from block_sparse_video_major_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_and_library_from_c(tmp_path):
    lib = L.LIB_PATH
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is missing: build it first")
    exe = tmp_path / "abi_from_c"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", str(exe), "-L", os.path.dirname(lib),
                    "-lvsa", "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok:") == 12
