"""Builds libamtk.so (the HIP kernels and the C-ABI) in-tree for gfx950.

Every .hip file under csrc/ is compiled by hipcc to an object, in parallel,
then linked into ``libamtk.so`` next to this file. Only the C-ABI symbols of
include/amtk.h are exported (-fvisibility=hidden elsewhere).

calib/*.hip (measurement kernels that are not part of the library: the L2
read ceiling the gather is reported against) link into ``libamtk_calib.so``.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libamtk.so")
CALIB_SRC = os.path.join(PKG, "calib")
CALIB_LIB = os.path.join(PKG, "libamtk_calib.so")
ARCH = os.environ.get("AMTK_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU instructions stay off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file flags. pass1_direct.hip: MFMA results in vector registers (its
# kernel may use the accumulation registers, where the compiler would
# otherwise put the results and copy each one out for the VALU).
FILE_FLAGS = {"pass1_direct.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(src):
    sub = "calib_" if os.path.dirname(src) == CALIB_SRC else ""
    obj = os.path.join(OBJ, sub + os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=True):
    """Compile every csrc/*.hip and link libamtk.so, and calib/*.hip into
    libamtk_calib.so. Always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    calib = sorted(os.path.join(CALIB_SRC, f) for f in os.listdir(CALIB_SRC)
                   if f.endswith(".hip"))
    jobs = min(len(srcs) + len(calib), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + calib))
    _link(objs[: len(srcs)], LIB)
    _link(objs[len(srcs):], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
