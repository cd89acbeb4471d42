"""Build the HIP library libmiattn.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmiattn.so")
PROBES_SRC = os.path.join(HERE, "probes", "peak_probes.hip")
PROBES_LIB = os.path.join(HERE, "libmiattn_probes.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(out: str, srcs, verbose: bool) -> None:
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
           *DEVICE_FLAGS, "-o", out + ".tmp", *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        msg = "\n".join(l for l in res.stderr.splitlines()
                        if "packed-fp32-ops" not in l)  # host pass does not know the feature
        if msg.strip():
            print(msg)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libmiattn.so, and the peak probes (a measurement aid
    of the benchmark) into libmiattn_probes.so.  Always recompiles."""
    _hipcc(LIB, sources(), verbose)
    _hipcc(PROBES_LIB, [PROBES_SRC], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
