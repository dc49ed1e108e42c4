"""Compile the HIP sources of librq_lut.so for gfx950 (hipcc, in-tree)."""
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "librq_lut.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# roctx: one named range per C-ABI call (shown by rocprofv3 --marker-trace)
LINK_LIBS = ["-L" + os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(out=LIB, extra=(), link_extra=()):
    """Compile every HIP source into `out` (always recompiles); returns `out`.

    Each source is compiled to an object in its own hipcc process (in parallel),
    then the objects are linked into the shared library."""
    tmp = out + ".tmp"
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    with tempfile.TemporaryDirectory(prefix="rq_build_") as objdir:
        objs, procs = [], []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            objs.append(obj)
            procs.append((src, subprocess.Popen(["hipcc", *HIPCC_FLAGS, *extra, *inc, "-c", src, "-o", obj])))
        failed = [src for src, pr in procs if pr.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, "hipcc -c " + " ".join(failed))
        subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp, *LINK_LIBS,
                        *link_extra], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
