"""Compile libqsa.so in-tree for gfx950 with hipcc (no JIT, no cache dir)."""
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libqsa.so")
# micro-benchmarks of the achievable MFMA and HBM rates (measurement only,
# never loaded by the path; built on request by build_probe())
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _link(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """libqsa.so: the QSA path."""
    _link(sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))), LIB, verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """libqsa_probe.so: the micro-benchmarks behind measure.py's `peaks`."""
    _link(sorted(glob.glob(os.path.join(PKG, "csrc", "probe", "*.hip"))), PROBE_LIB, verbose)
    return PROBE_LIB


if __name__ == "__main__":
    import sys
    print(build_probe(verbose=True) if "probe" in sys.argv[1:] else build(verbose=True))
