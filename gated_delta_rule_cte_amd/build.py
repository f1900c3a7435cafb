"""Build libgdn.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m gated_delta_rule_cte_amd.build

Each translation unit is compiled to an object under ``_build/`` in parallel,
then linked into ``gated_delta_rule_cte_amd/libgdn.so``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_tkg.hip", "gdn_cte.hip", "gdn_block.hip", "gdn_fused.hip", "gdn_block_cte.hip",
           "gdn_noalloc.hip", "gdn_blas.cpp"]
# measurement aids for bench.py, in a library of their own
CALIB_LIB = os.path.join(PKG, "libgdn_calib.so")
CALIB_SOURCES = ["gdn_calib.hip"]
# files whose MFMA accumulators stay in VGPRs (no per-iteration AGPR copies)
VGPR_MFMA = {"gdn_calib.hip"}
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; libgdn needs ROCm to build")
    return exe


def compile_flags(extra=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # no packed-fp32 instructions are generated anywhere in the library
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources: only the host code (argument validation, dispatch) is instrumented
# (each flag behind -Xarch_host); the GPU code is built as usual.  The
# sanitizer runtime is not linked in: the process that loads the library
# preloads clang's shared ASan runtime (tests/sanitize_host.py does).
HOSTSAN_LIB = os.path.join(PKG, "libgdn_hostsan.so")
HOSTSAN_DIR = os.path.join(PKG, "_build_hostsan")
HOSTSAN_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g")


def build(verbose: bool = True, extra_flags=(), out: str = LIB) -> str:
    _link(SOURCES, out, verbose, extra_flags)
    if out == LIB:
        _link(CALIB_SOURCES, CALIB_LIB, verbose, extra_flags)
    return out


def build_host_sanitized(verbose: bool = True) -> str:
    _link(SOURCES, HOSTSAN_LIB, verbose, HOSTSAN_FLAGS, build_dir=HOSTSAN_DIR)
    return HOSTSAN_LIB


def _link(sources, out, verbose, extra_flags, build_dir=BUILD_DIR):
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        vg = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] if src in VGPR_MFMA else []
        cmd = [cc, *compile_flags(extra_flags), *vg, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if msgs.strip() and verbose:
            print(msgs, flush=True)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(one, sources))
    tmp = out + ".tmp"
    libs = ["-lhipblaslt"] if "gdn_blas.cpp" in sources else []
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *libs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        build_host_sanitized(verbose="-q" not in sys.argv)
    else:
        build(verbose="-q" not in sys.argv)
