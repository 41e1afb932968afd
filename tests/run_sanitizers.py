"""CPU sanitizer run: the oracle and the HIP library's host code (argument validation, size
arithmetic, launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer, then the
CPU test suite, ``pytest -m "not gpu"``, run against those builds. Needs no GPU.

    python tests/run_sanitizers.py [extra pytest arguments]

Both builds use clang's sanitizer runtime (hipcc is clang; the oracle's sanitized build uses
ROCm's clang), which is preloaded into the Python process, since the interpreter itself is not
instrumented. Leak checking is off (the interpreter and torch keep allocations until exit)."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main() -> int:
    sys.path.insert(0, ROOT)
    from bcjr_soft_decoding_amd import build as hipbuild
    import oracle.oracle as orc

    print("building the sanitized library:", hipbuild.build(sanitize=True), flush=True)
    print("building the sanitized oracle:", orc.build(force=True, sanitize=True), flush=True)
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtimes:
        print("clang's AddressSanitizer runtime was not found under /opt/rocm/llvm", file=sys.stderr)
        return 2
    env = dict(os.environ)
    env.update({
        "BCJR_SANITIZE": "1",
        "LD_PRELOAD": runtimes[-1],
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q",
           "-p", "no:cacheprovider", *sys.argv[1:]]
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
