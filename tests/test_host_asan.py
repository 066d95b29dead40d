"""CPU: the C ABI's host code under AddressSanitizer.

Builds the host-ASan variant of the library (device code unchanged) and a
driver that calls every entry point through its validation paths; ASan
aborts the driver on any invalid host memory access, and the driver checks
each returned status.  No GPU is used: every call fails validation (or has
nothing to do) before a HIP call.
"""
import glob
import os
import subprocess

import pytest

from sparse_attention_token_absorb_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    lib = build.build(variant="asan")
    out = str(tmp_path_factory.mktemp("asan") / "asan_abi_driver")
    libdir = os.path.dirname(lib)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rt = glob.glob(os.path.join(rocm, "lib", "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no ASan runtime in this toolchain")
    rtdir = os.path.dirname(rt[0])
    cmd = [build.hipcc(), "-std=c++17", "-O1", *build.ASAN_HOST, "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "asan_abi_driver.cpp"), "-o", out, "-L", libdir, "-l:liblatentindex_asan.so",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rtdir}", "-Xarch_host", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_abi_validation_paths_under_asan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ok: 0 failures" in r.stdout
