"""Build libdllm.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdllm.so")
SOURCES = ["quantize.hip", "decode.hip", "qgemm.hip", "lmhead.hip", "attention.hip", "abi.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: never let the compiler form v_pk_{add,mul,fma}_f32.
# Correctly rounded f32 division is required for the Q8_K scale and is
# spelled out even though it is the HIP default.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Werror",
         "-Wno-unused-command-line-argument",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False) -> str:
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    errs = []
    for p, src in procs:
        _, err = p.communicate()
        # hipcc's host pass does not know the -packed-fp32-ops feature; that
        # warning is expected and harmless.
        err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errs.append(f"{src}:\n{err}")
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    if errs:
        raise RuntimeError("libdllm build failed:\n" + "\n".join(errs))
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
