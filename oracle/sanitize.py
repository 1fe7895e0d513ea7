"""Sanitizer pass over the CPU side: the oracle rebuilt with AddressSanitizer
and UndefinedBehaviorSanitizer, then the CPU test suite (``-m "not gpu"``)
run against that build in a child process.

    python oracle/sanitize.py

Host code only: nothing here builds or runs GPU code.  The sanitized copy is
written under ``_build/sanitize/`` and loaded through ``MXQ_ORACLE_LIB``;
the ASan runtime is preloaded into the child Python (leak checks off, since
the interpreter itself keeps memory until exit), and any report aborts the
run with a non-zero status.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxq_oracle.c")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "liboracle_asan_ubsan.so")


def runtime(name: str) -> str:
    return subprocess.check_output(["gcc", "-print-file-name=" + name],
                                   text=True).strip()


def main() -> int:
    os.makedirs(OUT_DIR, exist_ok=True)
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off",
         "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", SRC, "-o", LIB, "-lm"])
    env = dict(os.environ)
    env["MXQ_ORACLE_LIB"] = LIB
    pre = [runtime("libasan.so")]
    if env.get("LD_PRELOAD"):
        pre.append(env["LD_PRELOAD"])
    env["LD_PRELOAD"] = " ".join(pre)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"),
           "-m", "not gpu", "-q", "-p", "no:cacheprovider"]
    print("sanitized oracle:", LIB, flush=True)
    print(" ".join(cmd), flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
