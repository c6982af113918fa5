"""Build libpagedkv.so in-tree with hipcc for gfx950.

All HIP sources are compiled with packed-FP32 instruction selection turned
off and MFMA results kept in VGPRs; the host block manager is plain C++
compiled by the same driver.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpagedkv.so")
# The streaming-read probe: a measurement aid beside the library (not part of
# the decode path), loaded by bench.py only.
PROBE_LIB = os.path.join(HERE, "libpkvprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sources():
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.cpp")) + glob.glob(os.path.join(csrc, "*.hip")))


HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, out, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if msgs and (verbose or r.returncode):
        print("\n".join(msgs), file=sys.stderr)
    if r.returncode:
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(out + ".tmp", out)


def build_probe(verbose: bool = False) -> str:
    src = os.path.join(HERE, "probe", "stream_probe.hip")
    _run([HIPCC, *HIP_FLAGS, "-Wall", "-o", PROBE_LIB + ".tmp", src], PROBE_LIB, verbose)
    return PROBE_LIB


def build(verbose: bool = False, extra=()) -> str:
    build_probe(verbose)
    cmd = [HIPCC, *HIP_FLAGS,
           # MFMA accumulators in VGPRs: the decode kernel rescales them with
           # vector ops, which cannot read AGPRs without a copy each way.
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *extra, "-o", LIB + ".tmp", *sources()]
    _run(cmd, LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
