"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; no GPU code is instrumented and no kernel runs).

vsa_api.hip (every entry point's argument checks and the host helpers that
write caller arrays: the token order and the cube table) is compiled with the
sanitizers on its host side only, linked with the other objects of the
normal build into a separate library, and driven by the plain-C caller
tests/c/abi_from_c.c built with the same sanitizers.  A second caller that
hands vsa_perm_index an array one element short checks that the
instrumentation is live: the sanitizer must name that write.
"""
import os
import shlex
import subprocess

import pytest

from block_sparse_video_major_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
# sanitizers on the host side of the HIP translation unit only
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _objects():
    objs = sorted(os.path.join(B.BUILD, f) for f in os.listdir(B.BUILD) if f.endswith(".o")) \
        if os.path.isdir(B.BUILD) else []
    return [o for o in objs if os.path.basename(o) != "vsa_api.o"]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    objs = _objects()
    if len(objs) < 2 or not os.path.exists(CLANG):
        pytest.skip("needs the normal build's objects (__graft_entry__.build()) and ROCm's clang")
    d = tmp_path_factory.mktemp("hostsan")
    hipcc = B._hipcc()
    api_o = str(d / "vsa_api_san.o")
    subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-O1", "-std=c++17", "-fPIC", *shlex.split(HOST_SANITIZE),
                    "-c", os.path.join(B.CSRC, "vsa_api.hip"), "-o", api_o], check=True, capture_output=True)
    lib = str(d / "libvsa_san.so")
    subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, api_o, "-o", lib],
                   check=True, capture_output=True)

    def caller(src, name):
        exe = str(d / name)
        subprocess.run([CLANG, "-std=c99", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe, "-L", str(d), "-lvsa_san",
                        "-Wl,-rpath," + str(d)], check=True, capture_output=True)
        return exe
    return d, caller


def test_host_code_is_clean_under_sanitizers(sanitized):
    d, caller = sanitized
    exe = caller(os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "abi_san")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok:") == 12
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr


def test_sanitizer_is_live(sanitized):
    d, caller = sanitized
    src = open(os.path.join(ROOT, "tests", "c", "abi_from_c.c")).read()
    short = src.replace("int32_t perm[36 * 8];", "int32_t perm[36 * 8 - 1];")
    assert short != src
    bad = d / "short_array.c"
    bad.write_text(short)
    exe = caller(str(bad), "short_san")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode != 0
    assert "AddressSanitizer: stack-buffer-overflow" in r.stderr and "vsa_perm_index" in r.stderr, r.stderr[-2000:]
