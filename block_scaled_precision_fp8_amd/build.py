"""Build libbsfp8.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Every HIP source is compiled with packed-FP32 instruction generation disabled
(``-packed-fp32-ops``) and linked into one shared library next to this file."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsfp8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["api.hip", "quantize.hip", "gemm_fp8.hip", "gemm_fp8_big.hip", "gemm_fp8_outer.hip",
           "gemm_mxfp4.hip", "gemm_mx.hip"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    flags = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(HERE, "..", "include")]
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _drain(procs, verbose)
    _drain(procs, verbose)
    link = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _drain(procs, verbose):
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the device-only feature flag; that note is harmless
        lines = [l for l in text.splitlines() if "not a recognized feature" not in l]
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(lines))
        if verbose and lines:
            print("\n".join(lines))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
