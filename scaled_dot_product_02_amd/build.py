"""Build the HIP library libmiattn.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import tempfile

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


# Extra flags per source file.  The attention kernels take finite inputs (a documented
# contract), so their float max / min reductions need not quiet signalling NaNs: without
# -fno-honor-nans the compiler canonicalizes every MFMA result before its first v_max.
FILE_FLAGS = {
    "fa_fwd_bf16.hip": ["-fno-honor-nans"],
    "fa_fwd_persist.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, what: str, verbose: bool) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        msg = "\n".join(l for l in res.stderr.splitlines()
                        if "packed-fp32-ops" not in l)  # host pass does not know the feature
        if msg.strip():
            print(msg)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed building {what}")


# AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only (the device code is
# built exactly as in the normal library); the runtime is clang's shared one.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc(out: str, srcs, verbose: bool, libs=(), extra=(), link_extra=()) -> None:
    """Compile each source to an object in parallel, then link the shared library."""
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *extra]
    with tempfile.TemporaryDirectory(prefix="miattn_build_") as tmp:
        objs = [os.path.join(tmp, f"{i}_{os.path.basename(src)}.o") for i, src in enumerate(srcs)]
        jobs = [([HIPCC, *flags, *FILE_FLAGS.get(os.path.basename(src), ()), "-c", "-o", o, src],
                 os.path.basename(src)) for src, o in zip(srcs, objs)]
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, cmd, what, verbose) for cmd, what in jobs]:
                f.result()
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", out + ".tmp",
              *objs, *libs],
             os.path.basename(out), verbose)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libmiattn.so, and the peak probes (a measurement aid
    of the benchmark) into libmiattn_probes.so.  Always recompiles."""
    # rocBLAS runs the two projections of the multi-head module (mha.hip); an unresolved
    # symbol (a kernel whose host launch stub the compiler did not emit) fails the link
    # instead of the first launch
    strict = ("-Wl,--no-undefined",)
    _hipcc(LIB, sources(), verbose, libs=("-L/opt/rocm/lib", "-lrocblas"), link_extra=strict)
    _hipcc(PROBES_LIB, [PROBES_SRC], verbose, link_extra=strict)
    return LIB


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """The same library with the host code under ASan + UBSan, written to out_dir (for the
    CPU test run under sanitizers; load it with MIATTN_LIB and preload clang's ASan runtime)."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libmiattn_san.so")
    _hipcc(out, sources(), verbose, libs=("-L/opt/rocm/lib", "-lrocblas"), extra=HOST_SANITIZE,
           link_extra=("-fsanitize=address,undefined", "-shared-libasan"))
    return out


if __name__ == "__main__":
    import sys
    if len(sys.argv) == 3 and sys.argv[1] == "--sanitize":
        print(build_sanitized(sys.argv[2], verbose=True))
    else:
        print(build(verbose=True))
