"""Build the MSA HIP library (libmsa.so) in-tree for gfx950 with hipcc.

Run ``python -m block_sparse_attention_idx_amd.build`` (or call ``build()``).
Every call recompiles: object files go to ``_build/`` next to this file, the
library to ``libmsa.so`` in this package directory.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmsa.so")
SOURCES = ["msa_api.hip", "index_topk.hip", "attn.hip", "kl.hip", "bwd.hip"]
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in generated code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the GPU target feature; that line is noise
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)


# Host code of msa_api.hip (argument checks, planning, the C ABI) with
# AddressSanitizer and UBSan; device code and the other objects as built by
# build().  For running the ABI tests without a GPU under the sanitizers: load
# the result with MSA_LIBRARY and the ASan runtime (asan_runtime()) preloaded.
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libmsa_sanitized.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the sanitized library links against."""
    out = _run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"]).strip().splitlines()[-1]
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("the clang ASan runtime was not found")
    return out


def build_sanitized() -> str:
    objs = [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "msa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build()
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    obj = os.path.join(SANITIZE_DIR, "msa_api.o")
    _run([HIPCC, *COMMON_FLAGS, *SANITIZE_FLAGS, "-c", os.path.join(CSRC, "msa_api.hip"), "-o", obj])
    # the sanitizer hooks stay undefined in the library: the preloaded runtime provides them
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *objs, "-o", SANITIZE_LIB])
    return SANITIZE_LIB

