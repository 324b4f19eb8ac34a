"""Build libcgtp.so in-tree with hipcc for gfx950.

    python -m clebsch_gordan_tensor_cgtp_amd.build [--warm c1 c2 ...]

The host planner/ABI (C++) and the fixed kernels (HIP) are compiled into one
shared library next to this file.  ``--warm`` additionally creates the plans
of the named workloads so that their generated modules are compiled by hipRTC
now and stored in the on-disk cache (``jit_cache`` next to the library).
"""
import argparse
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libcgtp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

GPU_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.cpp"))) + sorted(glob.glob(os.path.join(csrc, "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-shared", *GPU_FLAGS,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *sources(), "-lhiprtc", "-ldl", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libcgtp.so")
    os.replace(tmp, LIB)
    return LIB


def warm(names):
    sys.path.insert(0, ROOT)
    from clebsch_gordan_tensor_cgtp_amd import binding, synth
    for name in names:
        for dtype in ("f32", "f64"):
            spec = synth.WORKLOADS[name]
            binding.plan_for(spec, dtype)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--warm", nargs="*", default=[])
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.v))
    if a.warm:
        warm(a.warm)


if __name__ == "__main__":
    main()
