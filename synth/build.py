"""Build the host (gcc/OpenMP) and device (hipcc, gfx950) fillers in-tree."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> None:
    src = os.path.join(_HERE, "csrc")
    host_cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                os.path.join(src, "synth_host.c"), "-o", os.path.join(_HERE, "_synth_host.so")]
    dev_cmd = [HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-ffp-contract=off", "-shared", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               os.path.join(src, "synth_fill.hip"), "-o", os.path.join(_HERE, "_synth_fill.so")]
    for cmd in (host_cmd, dev_cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
