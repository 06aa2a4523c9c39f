"""Build libmtpv.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m mtp_draft_verification_amd.build

Objects go to mtp_draft_verification_amd/_build/, the library to
mtp_draft_verification_amd/libmtpv.so. Packed fp32 instructions are disabled
for device code (the host pass warns that it does not know the feature; that
warning is harmless).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmtpv.so")
ARCH = os.environ.get("MTPV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "plan.hip", "lmhead.hip", "skinny.hip", "wide.hip", "headtile.hip", "verify.hip", "fuse.hip",
           "loss.hip", "ceiling.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-fvisibility=hidden",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


# The streaming kernel's load ring lives in registers only while its step loop is
# unrolled in full; its widest instances exceed the default size limit for that.
EXTRA_FLAGS = {"skinny.hip": ["-mllvm", "-pragma-unroll-threshold=65536"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=True):
    """Compile every source and link libmtpv.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
