"""Build libwa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libwa.so")
# Debug copy of the library whose attention kernel fills its LDS stages with
# NaN before every refill (WA_DEBUG_POISON); only a GPU test loads it.
LIB_POISON = os.path.join(PKG, "libwa_poison.so")
POISON_SRC = "k_attn_bf16.hip"

ARCH = "gfx950"
# Packed fp32 instructions stay off: plain fp32 arithmetic only.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


# Per-source flags.  The attention kernel asks for the VGPR form of the
# matrix-core instructions (its score tiles feed vector ALU work directly) and
# uses no AGPRs at all, so the whole 256-register budget of two wavefronts per
# SIMD goes to VGPRs.  It runs without the IEEE mode bit and assumes no NaNs
# (inputs are finite), so maxima of matrix-core results need no
# canonicalising instruction before each v_max.
EXTRA_FLAGS = {"k_attn_bf16.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee",
                                   "-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwa.so)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, poison: bool = False) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + (".poison.o" if poison else ".o"))
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + HIP_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + \
        (["-DWA_DEBUG_POISON"] if poison else []) + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libwa.so and its poison-checking debug
    copy libwa_poison.so; always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    poison_src = os.path.join(CSRC, POISON_SRC)
    with ThreadPoolExecutor(min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs))
        poison_obj = ex.submit(_compile, poison_src, True).result()
    _link(objs, LIB)
    _link([poison_obj if o.endswith(POISON_SRC + ".o") else o for o in objs], LIB_POISON)
    if verbose:
        print("built", LIB, "and", LIB_POISON)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
