"""The library's host code under AddressSanitizer (CPU only, no GPU involved).

Every csrc/*.hip file is rebuilt with the sanitizer on its host side only (device code
for gfx950 is compiled as usual), and tests/c/abi_check.c -- the plain-C consumer of
include/routed_moe.h that calls the size and layout queries and the validation paths,
which return before any HIP call -- runs against that build.  Any heap or stack misuse in
the host arithmetic (layouts, workspace sizing, argument checks) aborts the program."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.timeout(900)
def test_host_code_under_address_sanitizer(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc/clang not available")
    from routed_moe_layer_amd.build import COMMON_FLAGS, sources
    # host-side instrumentation only: each sanitizer flag goes to the host compilation
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"] + host_asan

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    lib = str(tmp_path / "libroutedmoe.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                        "-Xarch_host", "-fsanitize=address", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_check_asan")
    r = subprocess.run([CLANG, "-std=c99", "-Wall", "-fsanitize=address",
                        "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", str(tmp_path),
                        "-lroutedmoe", f"-Wl,-rpath,{tmp_path}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr
