"""Run the CPU test suite against host-sanitized builds (ASan + UBSan).

    python tests/sanitize_host.py [extra pytest args]

Builds gated_delta_rule_cte_amd/libgdn_hostsan.so (the C-ABI layer and every
launcher with AddressSanitizer and UndefinedBehaviorSanitizer on the host
code; GPU code unchanged) and oracle/liboracle_ref_san.so (the C oracle with
the same sanitizers, built with clang so that one sanitizer runtime serves
both), then runs ``pytest tests -m "not gpu"`` in a child process that
preloads clang's shared ASan runtime and points the binding and the oracle
loader at the sanitized builds.  Any sanitizer report aborts the run (UBSan
does not recover); leak checking is off (the Python interpreter itself is
not instrumented and keeps allocations alive at exit).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CLANG = "/opt/rocm/llvm/bin/clang"


def main(argv):
    from gated_delta_rule_cte_amd import build as gbuild
    lib = gbuild.build_host_sanitized(verbose=False)
    oracle_src = os.path.join(ROOT, "oracle", "gdn_ref.c")
    oracle_lib = os.path.join(ROOT, "oracle", "liboracle_ref_san.so")
    subprocess.check_call([CLANG, "-O1", "-g", "-fPIC", "-shared", "-std=c99", "-fopenmp",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", oracle_src, "-o", oracle_lib, "-lm"])
    runtime = subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    if not os.path.exists(runtime):
        raise SystemExit(f"ASan runtime not found: {runtime}")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "GDN_LIBRARY": lib,
        "GDN_ORACLE_LIBRARY": oracle_lib,
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *argv]
    print("sanitized run:", " ".join(cmd), flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
