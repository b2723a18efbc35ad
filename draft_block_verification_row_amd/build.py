"""Build libdspark_verify.so in-tree with hipcc for gfx950, and beside it
libdspark_stream_read.so (a plain streaming read: the measured read ceiling that
the throughput measurement compares the row-statistics pass with).

Usage: python -m draft_block_verification_row_amd.build
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("api.hip", "kernels.hip", "schedule.hip")]
LIB = os.path.join(PKG, "libdspark_verify.so")
READ_SOURCES = [os.path.join(PKG, "csrc", "stream_read.hip")]
READ_LIB = os.path.join(PKG, "libdspark_stream_read.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + sources + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile both HIP libraries (always recompiles) and return the sampler's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(READ_SOURCES, READ_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
