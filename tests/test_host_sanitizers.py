"""The host side of the library (argument checks, workspace arithmetic, the
ctypes binding) under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of the library is built with the sanitizers on its host code only (the
device code is built as usual and never launched here) under _build/asan/,
then the C-ABI tests run against that copy in a child process that preloads
the sanitizer runtime.  The copy is rebuilt only when a source, a header or
the flags change.
"""
import glob
import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_sparse_attention_causal_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libhysparse_asan.so")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# sanitizers on the host pass only
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         *SAN, f"-I{INCLUDE}", f"-I{CSRC}"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    deps = srcs + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + sorted(glob.glob(os.path.join(INCLUDE, "*.h")))
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for p in deps:
        h.update(p.encode())
        h.update(open(p, "rb").read())
    key = h.hexdigest()
    stamp = os.path.join(OUT, "sources.sha256")
    if os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == key:
        return LIB
    os.makedirs(OUT, exist_ok=True)
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]

    def cc(so):
        r = subprocess.run([HIPCC, *FLAGS, "-c", so[0], "-o", so[1]], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        list(ex.map(cc, zip(srcs, objs)))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, *objs, "-o", LIB],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(stamp, "w") as f:
        f.write(key)
    return LIB


CHILD = r"""
import ctypes, sys
assert hasattr(ctypes.CDLL(None), "__asan_init"), "sanitizer runtime not preloaded"
from hybrid_sparse_attention_causal_amd import binding as hb
hb.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py"]))
"""


@pytest.mark.skipif(not os.path.exists(HIPCC) or _runtime() is None, reason="hipcc or the ASan runtime missing")
def test_abi_under_host_sanitizers():
    lib = _build()
    # the copy really carries the instrumentation
    und = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in und and "__ubsan_handle" in und
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
