"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

  - the oracle (oracle/ugref.c) built with gcc's sanitizers: every oracle
    pin runs against it;
  - libug's host code (argument validation, the grouped-GEMV planner, size
    queries) built with the sanitizers on the host side only
    (-Xarch_host before each -fsanitize=; device code is unchanged): every
    C-ABI check runs against it.

Each run is a child Python process with the sanitizer runtime preloaded
(Python itself is not instrumented); leak checking is off (the interpreter
keeps its allocations), and any sanitizer report fails the test.  Skipped
where a runtime library is not installed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _runtime(cmd):
    try:
        path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(script, preload, arg):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", script, arg], env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out, out[-4000:]
    return out


PINS = r"""
import sys
sys.path.insert(0, %r); sys.path.insert(0, %r)
import oracle
import test_oracle_attention, test_oracle_backward, test_oracle_pins, test_oracle_sampler
n = 0
with oracle.use_library(sys.argv[1]):
    for mod in (test_oracle_pins, test_oracle_attention, test_oracle_sampler,
                test_oracle_backward):
        for name in sorted(dir(mod)):
            if name.startswith("test_") and name != "test_oracle_thread_count_invariance":
                getattr(mod, name)()
                n += 1
print("pins run:", n)
""" % (ROOT, os.path.join(ROOT, "tests"))


ABI = r"""
import sys
sys.path.insert(0, %r); sys.path.insert(0, %r)
from bitlinear_matmul_amd import ug
ug.LIB_PATH = sys.argv[1]
import test_abi
n = 0
for name in sorted(dir(test_abi)):
    if name.startswith("test_"):
        fn = getattr(test_abi, name)
        args = fn.__code__.co_varnames[:fn.__code__.co_argcount]
        fn(ug) if "ug" in args else fn()
        n += 1
print("abi checks run:", n)
""" % (ROOT, os.path.join(ROOT, "tests"))


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import build as obuild
    lib = str(tmp_path / "libugref_san.so")
    flags = [f for f in obuild.CFLAGS if f != "-O2"]
    subprocess.run(["gcc", *flags, "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    obuild.SRC, "-o", lib, "-lm"], check=True, capture_output=True)
    out = _run(PINS, asan, lib)
    assert "pins run:" in out


def test_libug_host_code_under_asan_ubsan(tmp_path):
    from bitlinear_matmul_amd import build as ubuild
    asan = _runtime([ubuild.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"])
    if asan is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    saved, saved_link = ubuild.FLAGS, ubuild.LINK_FLAGS
    ubuild.FLAGS = saved + san
    ubuild.LINK_FLAGS = []  # the sanitizer runtime is preloaded, not linked
    try:
        lib = ubuild.build_lib(ubuild.CSRC, str(tmp_path / "libug_san.so"))
    finally:
        ubuild.FLAGS, ubuild.LINK_FLAGS = saved, saved_link
    out = _run(ABI, asan, lib)
    assert "abi checks run:" in out
