"""Build libonela.so (the HIP library behind include/onela.h) and libonela_probe.so (the bench's bandwidth
probe, include/onela_probe.h) in-tree for gfx950 with hipcc."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "lib", "libonela.so")
PROBE_LIB = os.path.join(PKG, "lib", "libonela_probe.so")
SOURCES = ["onela_host.cpp", "context.hip", "step_generic.hip", "step_fused.hip", "fullstate.hip",
           "beam_select.hip", "materialize.hip", "prefill_mfma.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(sources, out_path, verbose):
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, "-o", tmp]
    for src in sources:
        path = os.path.join(CSRC, src)
        cmd += (["-x", "hip", path] if src.endswith(".cpp") else [path])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every source and link libonela.so and libonela_probe.so; returns libonela.so's path.  Always
    recompiles."""
    _compile(["hbm_probe.hip"], PROBE_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
