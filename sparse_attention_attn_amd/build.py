"""Build libattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc, and beside it
libattn_probes.so (the benchmark's read-rate probes; no attention entry point uses them).

Usage: python -m sparse_attention_attn_amd.build [--verbose]
The libraries land next to this file; object files go to sparse_attention_attn_amd/_build/.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libattn_probes.so")

SOURCES = ["fwd_dense.hip", "fwd_blocksparse.hip", "fwd_splitkv.hip", "sparse_index.hip", "api.cpp",
           "validate.cpp"]
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"
# Per-source extra flags for the dense kernel:
#  * no IEEE mode and no NaN semantics: its row maxima then lower to plain v_max3_f32 with no
#    operand quieting (inputs are finite; masked scores are -inf, which both settings keep);
#  * MFMA results in VGPRs: the scores feed VALU code directly, and the register allocator
#    parks the rarely touched output accumulators in AGPRs instead.
#  * fwd_splitkv.hip: MFMA results in VGPRs too. Its output accumulators are only rescaled on
#    the rare slow path, but with AGPR accumulators the compiler still moves all of them
#    through VGPRs around that branch on every tile.
EXTRA = {"fwd_dense.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans",
                           "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fwd_splitkv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def _common_flags():
    return [
        "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
        # Packed fp32 VALU forms are kept out of the generated code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _common_flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"] if src == "api.cpp" else []
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    err = "\n".join(x for x in res.stderr.splitlines() if "packed-fp32-ops" not in x)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(path)} failed:\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so and libattn_probes.so. Always rebuilds.
    Returns the path of libattn.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
