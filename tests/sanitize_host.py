"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer run (CPU only).

Builds sanitized copies of the oracle (clang, ``-fsanitize=address,undefined``)
and of libqlinear.so (hipcc with the sanitizers on the host pass only: each
``-fsanitize=`` follows ``-Xarch_host``; the gfx950 device code is built as
usual), then runs ``tests/test_oracle.py`` and ``tests/test_abi_host.py``
against them in a child pytest with the ASan runtime preloaded (Python itself
is not instrumented; leak detection is off because the interpreter keeps its
allocations to the end).  Any sanitizer report aborts the child and fails the
run.  Usage::

    python tests/sanitize_host.py            # build + run both files
    python tests/sanitize_host.py -k policy  # extra pytest arguments

Nothing here runs on a GPU: the ABI tests stop at the argument checks that
precede every HIP call.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "ggml_block_quant_amd", "_build", "sanitize")
LLVM = "/opt/rocm/llvm"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stderr[-4000:])


def asan_runtime() -> str:
    libs = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not libs:
        raise RuntimeError("clang's ASan runtime not found under " + LLVM)
    return libs[-1]


def build_oracle() -> str:
    out = os.path.join(OUT, "liboracle_san.so")
    _run([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall", "-shared", "-fPIC",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", out, "-lm"])
    return out


def build_qlinear() -> str:
    from ggml_block_quant_amd import build as B

    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run([B._hipcc(), *B.FLAGS, *san, "-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=len(B.SOURCES)) as ex:
        objs = list(ex.map(one, B.SOURCES))
    out = os.path.join(OUT, "libqlinear_san.so")
    _run([B._hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", out])
    return out


def main(extra) -> int:
    os.makedirs(OUT, exist_ok=True)
    print("building sanitized oracle and libqlinear ...", flush=True)
    with ThreadPoolExecutor(max_workers=2) as ex:
        fo, fq = ex.submit(build_oracle), ex.submit(build_qlinear)
        orc, qll = fo.result(), fq.result()
    env = dict(os.environ, ORACLE_LIB=orc, QLINEAR_LIB=qll, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:alloc_dealloc_mismatch=0:detect_odr_violation=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child must map the sanitized builds and the runtime, not the usual libraries
    probe = ("import oracle, ggml_block_quant_amd as q; oracle._L(); q.lib(); "
             "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if '_san.so' in l or 'rt.asan' in l}))")
    maps = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True).stdout
    print("mapped:", maps.strip(), flush=True)
    if not all(x in maps for x in (orc, qll, "rt.asan")):
        print("sanitized libraries not loaded", file=sys.stderr)
        return 1
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle.py"), os.path.join(ROOT, "tests", "test_abi_host.py"), *extra]
    print("running:", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
