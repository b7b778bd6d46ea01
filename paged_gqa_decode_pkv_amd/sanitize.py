"""Run the CPU checks of the host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

    python -m paged_gqa_decode_pkv_amd.sanitize [pytest args]

Builds the host-side sanitizer variant of libpkv.so (build.py --sanitize:
planner, policy, runner and the entry points' argument checks instrumented;
the kernels' device code as usual) and runs ``pytest -m "not gpu"`` over the
tests that call the library on the host (the C ABI, the planner, the policy),
in a child process that loads that variant (PKV_LIB_PATH) with the clang ASan
runtime preloaded.  Any report aborts the run (halt_on_error; leaks are not
checked, since the Python interpreter itself does not free everything at
exit).  CPU only: nothing here touches a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TESTS = ["tests/test_abi.py", "tests/test_policy.py"]


def asan_runtime(hipcc: str) -> str:
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def main(argv=None) -> int:
    from paged_gqa_decode_pkv_amd import build as B
    lib = B.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                          check=True).stdout
    if "__asan_init" not in syms or "__ubsan_handle" not in syms:
        raise RuntimeError(f"{lib} is not instrumented")
    env = dict(os.environ)
    env["PKV_LIB_PATH"] = lib
    env["LD_PRELOAD"] = asan_runtime(B._hipcc())
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    args = list(argv if argv is not None else sys.argv[1:]) or TESTS
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           *args]
    print("sanitized library:", lib, flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
