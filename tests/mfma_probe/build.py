"""Build the matrix-core probes (test instruments) into tests/mfma_probe/libmfmaprobe.so.

mfma_probe.hip (numerics) issues one of its instructions as inline assembly and
relies on the compiler's default register forms around it; rate_probe.hip
(issue rates) is compiled with matrix results in ordinary VGPRs, as the
library's GEMM kernels get them, so that its promotion loop carries no
accumulation-register copies."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmfmaprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = {"mfma_probe.hip": [], "rate_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    text = "\n".join(l for l in p.stdout.decode(errors="replace").splitlines()
                     if "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + text)
    if verbose and text:
        print(text)


def build(verbose: bool = False) -> str:
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(HERE, src.replace(".hip", ".o"))
        _run([HIPCC, *COMMON, *extra, "-c", os.path.join(HERE, src), "-o", obj], verbose)
        objs.append(obj)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
