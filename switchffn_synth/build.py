"""Build the generator's host (gcc + OpenMP) and device (hipcc, gfx950) fillers."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")


def build() -> None:
    host_out = os.path.join(HERE, "libswitchffn_synth_host.so")
    _run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall",
          "-I", CSRC, os.path.join(CSRC, "synth_host.c"), "-o", host_out + ".tmp"])
    os.replace(host_out + ".tmp", host_out)
    dev_out = os.path.join(HERE, "libswitchffn_synth_dev.so")
    _run([HIPCC, *HIP_FLAGS, "-I", CSRC, os.path.join(CSRC, "synth_fill.hip"),
          "-o", dev_out + ".tmp"])
    os.replace(dev_out + ".tmp", dev_out)


if __name__ == "__main__":
    build()
