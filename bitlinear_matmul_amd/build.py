"""Builds ``libug.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that matter for the results:
  -ffp-contract=off   no FMA contraction: every float op is rounded once,
                      as the fixed summation orders require;
  (defaults kept)     correctly rounded fp32 divide and sqrt, denormals kept;
  -packed-fp32-ops    off: hipcc may not form v_pk_*_f32 on its own.

Per-file flags (performance only): gemm.hip is compiled without the
post-register-allocation scheduler, which would otherwise regroup the
instruction order its K loop pins down (MFMAs interleaved one-for-one with
fragment reads and LDS-destination loads).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libug.so")
SOURCES = ["api.hip", "quant_act.hip", "absmean.hip", "pack.hip", "gemv_mfma.hip", "gemm.hip",
           "attention.hip", "sampler.hip", "backward.hip", "probe.hip"]
ARCH = os.environ.get("UG_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# gemm.hip: keep the K loop's pinned issue order (no post-RA rescheduling).
# gemv_mfma.hip: the hardware preloads the first two kernel-argument dwords
# (the block table pointer) into SGPRs, saving a memory round trip at the
# start of every block of a decode launch.
# -z defs: a symbol left undefined (say a kernel whose launch stub the host
# pass did not emit) fails the link instead of the first load.  (A build
# with host sanitizers links without it: their runtime is preloaded.)
LINK_FLAGS = ["-Wl,-z,defs"]
FILE_FLAGS = {"gemm.hip": ["-mllvm", "-enable-post-misched=false"],
              "gemv_mfma.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=2"]}


def sources(src_dir=CSRC):
    return [os.path.join(src_dir, s) for s in SOURCES]


def inputs_mtime():
    files = sources() + [os.path.join(CSRC, "ug_internal.h"),
                         os.path.join(HERE, "..", "include", "ug.h"),
                         os.path.abspath(__file__)]
    return max(os.path.getmtime(f) for f in files)


def build_lib(src_dir, out, verbose=False):
    """Compile every source of src_dir to an object (in parallel), then link
    the shared library `out`.  Raises RuntimeError with hipcc's output on
    failure."""
    with tempfile.TemporaryDirectory(prefix="ugbuild") as tmpd:
        def compile_one(name):
            obj = os.path.join(tmpd, name + ".o")
            cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(name, []), "-c",
                   os.path.join(src_dir, name), "-o", obj]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            return obj, subprocess.run(cmd, capture_output=True, text=True)
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
            results = list(ex.map(compile_one, SOURCES))
        for obj, r in results:
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError("hipcc failed compiling " + os.path.basename(obj))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *LINK_FLAGS,
               *[o for o, _ in results], "-o", tmp]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking " + os.path.basename(out))
        os.replace(tmp, out)
    return out


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libug.so in-tree; returns its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= inputs_mtime():
        return LIB
    return build_lib(CSRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
