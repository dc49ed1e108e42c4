"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds, both with clang and the shared sanitizer runtime:
- the host code of librq_lut.so (argument checks, workspace sizing, the
  planners, launch sequencing), compiled for the host only: with no GPU nothing
  launches, and the sanitizers do not instrument GPU code anyway;
- the CPU oracle, without OpenMP (its parallel loops are over independent rows,
  so a serial run computes the same values).
The runtime is preloaded into a fresh Python that runs pytest -m "not gpu" on
the chosen test files, loading the two builds through RQ_LUT_LIB and
RQ_ORACLE_LIB. Any sanitizer report ends that run with a non-zero status.

Usage: python tests/sanitize_run.py [test files or pytest options ...]
(default: every test file, -m "not gpu"). Builds and sanitizer reports go to
tests/_sanitize/ (not tracked); a failing run prints the reports.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "_sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")

sys.path.insert(0, ROOT)

# Host-only sanitizer flags: each -fsanitize= sits right after -Xarch_host so that
# no device code is ever built with it.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan"]
ORACLE_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
              "-shared-libsan", "-g", "-Wno-unknown-pragmas"]

DEFAULT_TESTS = ["tests"]


def runtime():
    """The shared ASan runtime of ROCm's clang (it carries UBSan's handlers too)."""
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under " + ROCM)
    return hits[-1]


def build():
    from lut_logits_amd import build as hip_build
    from oracle import build as oracle_build

    os.makedirs(OUT, exist_ok=True)
    lib = hip_build.build(out=os.path.join(OUT, "librq_lut_san.so"), extra=HOST_SAN)
    orc = oracle_build.build(out=os.path.join(OUT, "liboracle_san.so"), extra=ORACLE_SAN, cc=CLANG, openmp=False)
    return lib, orc


def run(args):
    lib, orc = build()
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime() + (":" + pre if pre else "")
    # reports go to files: pytest holds the test's stderr, and a halted run never prints it
    for f in glob.glob(os.path.join(OUT, "report.*")):
        os.remove(f)
    log = os.path.join(OUT, "report")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:exitcode=86:log_path={log}"   # Python's own allocations are not leaks
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:exitcode=87:log_path={log}"
    env["RQ_LUT_LIB"], env["RQ_ORACLE_LIB"] = lib, orc
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *(args or DEFAULT_TESTS)]
    rc = subprocess.run(cmd, cwd=ROOT, env=env).returncode
    reports = sorted(glob.glob(log + ".*"))
    for f in reports:
        with open(f) as fh:
            print(f"--- {f}\n" + "".join(fh.readlines()[:40]), file=sys.stderr)
    return rc if rc != 0 or not reports else 88


if __name__ == "__main__":
    sys.exit(run(sys.argv[1:]))
