"""Build libswitchffn.so (the C-ABI library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libswitchffn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "router.hip", "dispatch.hip", "ffn.hip", "bwd.hip", "noalloc.hip"]
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         # Packed fp32 instructions stay off: the compiler must not form them.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return out


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD, defines=(),
          csrc: str = CSRC) -> str:
    """Compile and link the library (defines: extra -D options for tuning builds)."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        jobs.append(([HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c",
                      os.path.join(csrc, src), "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o in jobs],
          "-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
