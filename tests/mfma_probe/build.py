"""Build the matrix-core probe (test instrument) into tests/mfma_probe/libmfmaprobe.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmfmaprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "mfma_probe.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    text = "\n".join(l for l in p.stdout.decode(errors="replace").splitlines()
                     if "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for mfma_probe.hip:\n" + text)
    if verbose and text:
        print(text)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
