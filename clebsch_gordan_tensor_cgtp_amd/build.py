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

ROCM_INC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
GPU_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.cpp"))) + sorted(glob.glob(os.path.join(csrc, "*.hip")))


def _compile(args):
    cmd, verbose = args
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stdout + r.stderr


def build(verbose: bool = False) -> str:
    """Host C++ sources are compiled as plain C++, the .hip sources for gfx950; then linked."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    jobs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", *GPU_FLAGS, *inc, "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, *inc, "-c", src,
                   "-o", obj]
        jobs.append((cmd, verbose))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for rc, log in ex.map(_compile, jobs):
            if rc != 0:
                sys.stderr.write(log)
                raise RuntimeError("hipcc failed building libcgtp.so")
    tmp = LIB + f".tmp{os.getpid()}"
    rc, log = _compile(([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-lhiprtc", "-ldl", "-o", tmp],
                        verbose))
    if rc != 0:
        sys.stderr.write(log)
        raise RuntimeError("linking libcgtp.so failed")
    os.replace(tmp, LIB)
    return LIB


def warm(names):
    """Create the named workloads' plans (both dtypes) and build the modules that are otherwise
    compiled on first use: the backward of uvw plans (batched or convolution)."""
    sys.path.insert(0, ROOT)
    from clebsch_gordan_tensor_cgtp_amd import binding, synth
    for name in names:
        for dtype in ("f32", "f64"):
            spec = {**synth.WORKLOADS, **synth.EXTRA_WORKLOADS}[name]
            plan = binding.plan_for(spec, dtype)
            if spec.mode != "uvw":
                continue
            if hasattr(spec, "n_edges"):
                plan.conv_uvw_backward_source(0)
            else:
                plan.uvw_backward_source()


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
