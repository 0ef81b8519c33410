"""Compile the HIP library ``libpolykv.so`` for gfx950, in-tree.

Usage: ``python -m agent_q8_quant_amd.build`` (or ``build()`` from Python). Every call
recompiles; objects go to ``agent_q8_quant_amd/_build/`` and the library next to this
file, where the binding loads it.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpolykv.so")
SOURCES = ["host.cpp", "compress.hip", "attend.hip", "attend_mfma.hip", "attend_tail.hip", "dequant.hip", "project.hip"]

# -packed-fp32-ops: no packed fp32 VALU instructions in device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]


# per-file extras: the value compressor keeps matrix-core results in ordinary vector
# registers (its compares read them directly)
FILE_FLAGS = {"compress.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "project.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([hipcc] + DEVICE_FLAGS + FILE_FLAGS.get(src, []) + inc + lang +
             ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
