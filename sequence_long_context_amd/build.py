"""Build libulysses.so (gfx950) in-tree with hipcc.

Packed-fp32 instructions are disabled for the device code: hipcc forms them by
itself from ordinary float code, and the kernels here do not need them.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libulysses.so")
SOURCES = ["api.hip", "layout.hip", "attention_bf16.hip", "attention_bwd_bf16.hip",
           "attention_f32.hip", "merge.hip", "scratch.hip"]
ARCH = "gfx950"


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = (["hipcc"] + hipcc_flags() + ["-shared"] +
           [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
