"""Runs the CPU test suite (-m "not gpu") under AddressSanitizer + UndefinedBehaviorSanitizer.

Two runs, because gcc and clang bring different sanitizer runtimes and only one can be loaded:
  1. the oracle built by gcc with -fsanitize=address,undefined (liborc_moe_san.so), gcc's libasan
     preloaded;
  2. the library's host code (argument checks, sizing, launchers) built by hipcc with the same
     sanitizers on the host side only (libmoe_rocm_san.so), clang's shared ASan runtime preloaded.
Leak detection is off (the Python interpreter and torch are not instrumented and keep allocations
alive until exit). Usage: python tests/sanitizers.py [--no-build] [extra pytest args]
Exit status: that of the first failing run, else 0. pytest captures only Python-level output
(--capture=sys), so a sanitizer report written to file descriptor 2 reaches the terminal.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime(cmd):
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()


def main() -> int:
    args = [a for a in sys.argv[1:] if a != "--no-build"]
    if "--no-build" not in sys.argv:
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__.build(sanitize=True)
    gcc_asan = runtime(["gcc", "-print-file-name=libasan.so"])
    clang_asan = runtime(["/opt/rocm/lib/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"])
    base = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    runs = [("oracle (gcc ASan+UBSan)", dict(base, MOE_SANITIZE_ORACLE="1", LD_PRELOAD=gcc_asan)),
            ("library host code (clang ASan+UBSan)", dict(base, MOE_SANITIZE_LIB="1", LD_PRELOAD=clang_asan))]
    for name, env in runs:
        print(f"[sanitizers] {name}: pytest -m 'not gpu'", flush=True)
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m", "not gpu",
                            "-p", "no:cacheprovider", "--capture=sys", *args], cwd=ROOT, env=env)
        if r.returncode != 0:
            print(f"[sanitizers] {name}: FAILED (exit {r.returncode})", flush=True)
            return r.returncode
    print("[sanitizers] both runs passed", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
