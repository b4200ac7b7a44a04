"""Build the seeded input generator: a host library (gcc, OpenMP) and a device
library (hipcc, gfx950).  Both implement the definition in synth.h."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    host = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
            "-shared", "-Wall", "-o", HOST_LIB + ".tmp", os.path.join(HERE, "synth_host.c"), "-lm"]
    dev = ["hipcc", *HIP_FLAGS, "-o", DEV_LIB + ".tmp", os.path.join(HERE, "synth_dev.hip")]
    for cmd, out in ((host, HOST_LIB), (dev, DEV_LIB)):
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose=True)
