"""Build libkvcodec.so in-tree with hipcc for gfx950 (no GPU needed)."""

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkvcodec.so")

# -ffp-contract=off: the codec's float steps are defined operation by
# operation; no multiply-add may be fused behind our back.
# -packed-fp32-ops off: no packed fp32 instructions are generated.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


# streaming bandwidth probes of the benchmark (not part of the codec ABI)
PROBE_SRC = os.path.join(PKG, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "libkvprobe.so")


def _hipcc(srcs, out, verbose, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + list(extra) + list(srcs) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        sys.stderr.write(errs + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    if verbose and errs:
        print(errs)
    os.replace(tmp, out)
    return out


def build(verbose=False, extra=()):
    """libkvcodec.so (the codec) and libkvprobe.so (the benchmark's probes)."""
    _hipcc(sources(), LIB_PATH, verbose, extra)
    _hipcc([PROBE_SRC], PROBE_LIB, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
