"""Build libulysses.so (gfx950) in-tree with hipcc.

Packed-fp32 instructions are disabled for the device code: hipcc forms them by
itself from ordinary float code, and the kernels here do not need them.  Each
source is compiled on its own (some take extra flags, FILE_FLAGS), then linked.
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libulysses.so")
SOURCES = ["api.hip", "layout.hip", "attention_bf16.hip", "attention_bf16_chs.hip",
           "attention_bwd_bf16.hip", "attention_f32.hip", "merge.hip", "scratch.hip"]
# the chain-split kernels are faster with this instruction-scheduler strategy, the
# 256-row kernels slower (see the header of attention_bf16_chs.hip)
FILE_FLAGS = {"attention_bf16_chs.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}
ARCH = "gfx950"


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    objdir = tempfile.mkdtemp(prefix="uly_build_")
    try:
        objs = []
        for s in SOURCES:
            obj = os.path.join(objdir, s.replace(".hip", ".o"))
            _run(["hipcc"] + hipcc_flags() + FILE_FLAGS.get(s, []) +
                 ["-c", os.path.join(CSRC, s), "-o", obj], verbose)
            objs.append(obj)
        _run(["hipcc", "--offload-arch=" + ARCH, "-shared"] + objs + ["-o", tmp], verbose)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
