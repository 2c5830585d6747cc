"""Build libattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m exact_scaled_dot_sdpa_amd.build [-v]

Every .hip file under csrc/ is compiled by hipcc for --offload-arch=gfx950 and
linked into exact_scaled_dot_sdpa_amd/libattn.so.  Packed fp32 instructions are
disabled for the device code (-target-feature -packed-fp32-ops).
"""
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# The sources each logical kernel is built from (csrc/ file names).
KERNEL_SOURCES = {
    "prefill": ("prefill_bf16.hip", "kernels.h"),
    "decode": ("decode.hip", "kernels.h"),
    "bwd": ("bwd_bf16.hip", "kernels.h"),
    "fp8": ("prefill_fp8.hip", "kernels.h"),
}


def source_digest(kernel=None) -> str:
    """Digest of the kernel sources: all of csrc/*.hip, *.h, or only those of
    one logical kernel ("prefill", "decode", "bwd").  Stored hardware-counter figures
    carry it, so that figures taken on other kernels are not reused."""
    if kernel is None:
        names = [n for n in sorted(os.listdir(CSRC)) if n.endswith((".hip", ".h"))]
    else:
        names = sorted(KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def command(out=LIB, extra=()):
    return [
        "hipcc", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall",
        *extra, "-o", out, *sources(),
    ]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = ["-Rpass-analysis=kernel-resource-usage"] if "--usage" in sys.argv else []
    print(build(verbose="-v" in sys.argv[1:], extra=extra))
