"""Build libh3attn.so in-tree for gfx950.

The HIP sources are compiled with hipcc; the host coordinate builder with g++
and -ffp-contract=off (its binary64 formula must not be fused).  Objects go to
_build/ next to the package; the library lands in the package directory.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libh3attn.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["h3attn_api.hip", "rope_kernel.hip", "attn_fwd.hip", "adaln_kernel.hip", "pack_kernel.hip",
               "gemm_kernel.hip"]
HOST_SOURCES = ["coords.cpp"]

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-I" + INCLUDE]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 device feature; drop that notice only
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose=False, save_temps=False, out=None, extra_flags=(), build_dir=None, csrc=None):
    """Compile every source and link the library (default: libh3attn.so in the package).

    extra_flags are appended to the HIP compile lines (e.g. -D overrides of the
    kernels' tile constants); out, build_dir and csrc redirect the products and
    the source directory.  Always rebuilds.
    """
    out = out or LIB
    bdir = build_dir or BUILD
    src_dir = csrc or CSRC
    os.makedirs(bdir, exist_ok=True)
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        extra = ["-save-temps=obj"] if save_temps else []
        jobs.append([HIPCC] + HIP_FLAGS + list(extra_flags) + extra + ["-c", os.path.join(src_dir, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        jobs.append(["g++"] + HOST_FLAGS + ["-c", os.path.join(src_dir, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for log in ex.map(_run, jobs):
            if verbose and log.strip():
                print(log)
    objs = [os.path.join(bdir, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
