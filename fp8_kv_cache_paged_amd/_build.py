"""Build the HIP library (libmla_fp8.so) in-tree for gfx950 with hipcc.

Kernels and the C-ABI host layer are compiled in one hipcc invocation per
translation unit and linked into a shared library next to this file. The
library exports only the symbols declared in include/mla_fp8.h.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmla_fp8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ASM_DIR = os.path.join(PKG_DIR, "_asm")   # device assembly of the last build
ARCH = os.environ.get("MLA_FP8_ARCH", "gfx950")

SOURCES = ["mla_decode.hip", "mla_decode_ws.hip", "quantize.hip", "probes.hip", "noalloc.hip", "host.cpp"]

# Packed fp32 VALU instructions are switched off for all device code: hipcc
# would otherwise form v_pk_* fp32 ops from float2 arithmetic by itself.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
                "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compile every source and link libmla_fp8.so; returns the library path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="mla_fp8_build_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            # .hip sources also keep their gfx950 assembly (-save-temps), which
            # the wait-state check in tests/ reads
            lang = ["-x", "hip", "-save-temps=obj"] if src.endswith(".hip") else []
            cmds.append([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        os.makedirs(ASM_DIR, exist_ok=True)
        for src in SOURCES:
            if not src.endswith(".hip"):
                continue
            stem = src[: -len(".hip")]
            cands = [f for f in os.listdir(tmp) if f == f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s"]
            if len(cands) != 1:
                raise RuntimeError(f"device assembly of {src} not found among the build temporaries")
            shutil.copyfile(os.path.join(tmp, cands[0]), os.path.join(ASM_DIR, src + ".s"))
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        # atomic replace so that a running process never sees a half-written file
        staged = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
