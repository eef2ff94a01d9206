"""Compile the synthetic input generators: libsynth.so (gcc) and libsynth_gpu.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False):
    host_out = os.path.join(HERE, "libsynth.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
           os.path.join(HERE, "synth.c"), "-o", host_out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(host_out + ".tmp", host_out)

    gpu_out = os.path.join(HERE, "libsynth_gpu.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "synth_gpu.hip"), "-o", gpu_out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
    os.replace(gpu_out + ".tmp", gpu_out)
    return host_out, gpu_out


if __name__ == "__main__":
    print(build(verbose=True))
