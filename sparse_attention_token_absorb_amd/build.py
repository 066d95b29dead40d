"""Build liblatentindex.so (gfx950) from the HIP/C++ sources in csrc/.

    python -m sparse_attention_token_absorb_amd.build

Each source compiles with hipcc --offload-arch=gfx950 into _build/, then the
objects link into a shared library next to this file.  hipcc cross-compiles,
so no GPU is needed.  Packed fp32 VALU instructions are disabled for device
code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblatentindex.so")
SOURCES = ["api.cpp", "timing.cpp", "append.hip", "absorb.hip", "score.hip", "select.hip", "fp8.hip", "rope.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Host-side AddressSanitizer build (variant "asan"): the host code of every
# source is instrumented; device code is built as usual (GPU sanitizers are
# not used).  Each -fsanitize flag applies to the host pass only.
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
BUILD_ASAN = os.path.join(HERE, "_build_asan")
LIB_ASAN = os.path.join(BUILD_ASAN, "liblatentindex_asan.so")
# Instrumented build (variant "phases"): the decode scoring kernels record
# per-wave phase timestamps (li_phase_records); everything else is the same.
BUILD_PHASES = os.path.join(HERE, "_build_phases")
LIB_PHASES = os.path.join(BUILD_PHASES, "liblatentindex_phases.so")
_OUT = {None: (BUILD, LIB), "asan": (BUILD_ASAN, LIB_ASAN), "phases": (BUILD_PHASES, LIB_PHASES)}


def _flags(variant=None):
    # MFMA accumulators in VGPRs: the decode kernels' epilogue then reads them
    # without a v_accvgpr_read per element (32 per tile), which a wave alone
    # on its SIMD would otherwise spend before issuing its next loads.
    f = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
    if variant == "asan":
        f += ASAN_HOST
    elif variant == "phases":
        f += ["-DLI_PHASE_PROBE=1"]
    return f


def _compile(src: str, variant=None) -> str:
    out_dir = _OUT[variant][0]
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(variant), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, variant=None) -> str:
    """Build liblatentindex.so (variant None), the host-ASan library
    _build_asan/liblatentindex_asan.so (variant "asan") or the instrumented
    _build_phases/liblatentindex_phases.so (variant "phases")."""
    if variant not in _OUT:
        raise ValueError(f"unknown build variant {variant!r}")
    out_dir, lib = _OUT[variant]
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, variant), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if variant == "asan":
        cmd += ["-Xarch_host", "-fsanitize=address", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, variant=sys.argv[1] if len(sys.argv) > 1 else None)
    sys.exit(0)
