"""Compile the HIP library libswitch_layer.so for gfx950 (in-tree, explicit hipcc)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libswitch_layer.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["switch_layer.hip", "router.hip", "assign.hip", "move.hip", "gemm.hip", "ffn.hip",
           "backward.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


# attainable-peak probes of the measurement (a library of their own)
PEAKS_LIB = os.path.join(LIBDIR, "libswitch_peaks.so")


def _hipcc(srcs, out, verbose):
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o",
           out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    _hipcc([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose)
    _hipcc([os.path.join(CSRC, "peaks.hip")], PEAKS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
