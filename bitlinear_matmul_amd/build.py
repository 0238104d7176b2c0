"""Builds ``libug.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that matter for the results:
  -ffp-contract=off   no FMA contraction: every float op is rounded once,
                      as the fixed summation orders require;
  (defaults kept)     correctly rounded fp32 divide and sqrt, denormals kept;
  -packed-fp32-ops    off: hipcc may not form v_pk_*_f32 on its own.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libug.so")
SOURCES = ["api.hip", "quant_act.hip", "absmean.hip", "pack.hip", "gemv_mfma.hip", "gemm.hip"]
ARCH = os.environ.get("UG_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def inputs_mtime():
    files = sources() + [os.path.join(CSRC, "ug_internal.h"),
                         os.path.join(HERE, "..", "include", "ug.h")]
    return max(os.path.getmtime(f) for f in files)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libug.so in-tree; returns its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= inputs_mtime():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libug.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
