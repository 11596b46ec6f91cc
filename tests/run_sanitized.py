"""Run the host-only tests (-m "not gpu") with the oracle and the library's
host code built under AddressSanitizer and UndefinedBehaviorSanitizer.

    python tests/run_sanitized.py [extra pytest args]

Builds oracle/libptq1_oracle_asan.so and _build/sanitize/libptq1.so,
preloads gcc's sanitizer runtimes into a child pytest process, points the
oracle and the binding at the instrumented builds (PTQ1_ORACLE_LIB,
PTQ1_LIB) and exits with pytest's status.  Any sanitizer report aborts the
run (halt_on_error).  The input generator's host side is numpy (nothing to
instrument); no GPU code is instrumented."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path):
        raise RuntimeError(f"gcc does not provide {name}")
    return path


def main() -> int:
    import oracle
    from ternary_weight_ptq1_amd import build as b

    olib = oracle.build(force=True, sanitize=True)
    plib = b.build_sanitized(verbose=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join([runtime("libasan.so"), runtime("libubsan.so")])
    # Python and the libraries it loads are not instrumented: leaks at exit and
    # their allocator mismatches are not this code's; errors in the
    # instrumented code still abort the run
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1:alloc_dealloc_mismatch=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PTQ1_ORACLE_LIB"] = olib
    env["PTQ1_LIB"] = plib
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *sys.argv[1:]]
    print("running:", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
