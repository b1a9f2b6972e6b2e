"""Build the gfx950 shared libraries in-tree.

* ``sparse_long_context_block_amd/libsgqa.so`` -- the product library
  (``csrc/*.hip``), C ABI in ``include/sgqa.h``;
* ``synth/libsynth.so`` -- the device twin of the seeded input generator.

Every .hip file is compiled separately with hipcc for gfx950 (object files
under ``_build/``) and the objects are linked into the shared library.
``python -m sparse_long_context_block_amd.build`` builds both.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

LIB_SGQA = os.path.join(PKG, "libsgqa.so")
LIB_SYNTH = os.path.join(ROOT, "synth", "libsynth.so")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libsgqa.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _compile(src: str, obj: str, includes) -> str:
    cmd = [_hipcc(), *HIP_FLAGS, *(f"-I{i}" for i in includes), "-c", src, "-o", obj]
    return _run(cmd)


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)


def build_lib(sources, out: str, includes, tag: str, verbose: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, tag), exist_ok=True)
    objs = [os.path.join(BUILD, tag, os.path.basename(s) + ".o") for s in sources]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        futs = [ex.submit(_compile, s, o, includes) for s, o in zip(sources, objs)]
        for f in futs:
            log = f.result()
            if verbose and log.strip():
                print(log)
    _link(objs, out)
    return out


def sgqa_sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> None:
    """Compile libsgqa.so and libsynth.so for gfx950 (always recompiles)."""
    build_lib(sgqa_sources(), LIB_SGQA, [INCLUDE, CSRC], "sgqa", verbose)
    build_lib([os.path.join(ROOT, "synth", "gen.hip")], LIB_SYNTH, [], "synth", verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB_SGQA)
    print(LIB_SYNTH)
