"""Run the CPU test suite (-m "not gpu") with the host code under ASan and
UBSan: builds the sanitized oracle, host layer and C program
(build_sanitized.py), preloads the sanitizer runtimes into the Python process
and sets RMSQ_SANITIZE=1 so that tests/conftest.py loads the sanitized
libraries.  Any sanitizer report aborts the run.

    python tests/sanitize/run_sanitized.py [extra pytest arguments]
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, HERE)
import build_sanitized  # noqa: E402


def runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def main() -> int:
    build_sanitized.build(verbose=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join([runtime("libasan.so"), runtime("libubsan.so")] +
                                 ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    # the interpreter and its extension modules are not instrumented: leak
    # reports would be theirs; link order is the preload's
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["RMSQ_SANITIZE"] = "1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q", *sys.argv[1:]]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
