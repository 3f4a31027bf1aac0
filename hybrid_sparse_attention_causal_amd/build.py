"""Build libhysparse.so (the HIP kernels + C ABI) for gfx950, in-tree.

    python -m hybrid_sparse_attention_causal_amd.build

Every HIP source under csrc/ is compiled with hipcc for gfx950 (in parallel),
then linked into hybrid_sparse_attention_causal_amd/libhysparse.so.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhysparse.so")

ARCH = os.environ.get("HS_OFFLOAD_ARCH", "gfx950")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Kernels allowed to use per-lane scratch (register spills). Spills on the hot
# kernels cost several times their run time, so any other kernel that spills
# fails the build. Only fp32-input variants, which are correctness paths and
# not tuned, are listed.
SCRATCH_ALLOWED = {
    "_ZN2hs24sparse_prefill_pp_kernelILi0ELi64ELi2EEEvNS_17SparsePrefillArgsE",
    "_ZN2hs21sparse_prefill_kernelILi0ELi128ELi1ELi8ELi2EEEvNS_17SparsePrefillArgsE",
}
_REMARK = "kernel-resource-usage"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _spills(remarks: str) -> dict:
    """Kernel name -> scratch bytes per lane, from the resource-usage remarks."""
    found, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)):
            found[name] = int(m.group(1))
    return found


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(so):
        src, obj = so
        out = _run([HIPCC, *CFLAGS, f"-Rpass-analysis={_REMARK}", "-c", src, "-o", obj])
        spills = {k: v for k, v in _spills(out).items() if k not in SCRATCH_ALLOWED}
        if spills:
            raise RuntimeError(f"{os.path.basename(src)}: kernels spill to scratch "
                               f"(bytes/lane): {spills}")
        return "\n".join(l for l in out.splitlines() if _REMARK not in l)

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        outs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    # every kernel launch stub must be defined in the library itself
    missing = [l.split()[-1] for l in _run(["nm", "-D", "--undefined-only", tmp]).splitlines()
               if "__device_stub__" in l]
    if missing:
        raise RuntimeError(f"libhysparse.so leaves kernel launch stubs undefined: {missing[:4]}")
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
