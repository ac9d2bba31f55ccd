"""Build the HIP library libpa_mi355x.so for gfx950 (in-tree, next to this file), and
the benchmark's HBM read probe libpa_hbm_probe.so (a measurement helper, no part of
the attention path).

hipcc cross-compiles without a GPU.  Packed-fp32 instruction selection is switched
off for device code; hipcc's host pass warns that it does not know that feature,
which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpa_mi355x.so")
PROBE_LIB = os.path.join(HERE, "libpa_hbm_probe.so")
SOURCES = ["pa_api.cpp", "pa_alloc.cpp", "pa_validate.cpp", "pa_decode.hip", "pa_append.hip", "pa_prefill.hip"]
ARCH = "gfx950"


def hip_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build_library(out=LIB, verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *hip_flags(), "-c", "-x", "hip", path, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        if verbose:
            sys.stderr.write(res.stderr)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_probe(out=PROBE_LIB):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *hip_flags(), "-shared", "-x", "hip",
           os.path.join(CSRC, "hbm_read_probe.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed on hbm_read_probe.hip")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    print(build_probe())
