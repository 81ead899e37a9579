"""Builds libsparse_attn.so (all HIP sources, gfx950) in-tree.

    python -m block_sparse_attention_scores_amd.build [--sanitize]

Objects go to _build/ at the repository root; the library to
block_sparse_attention_scores_amd/lib/.  Every call recompiles.

--sanitize builds a second library, _build/san/libsparse_attn.so, whose host
code (argument validation, workspace carving, launch sequencing) is
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; device
code is built as usual.  It is loaded by the CPU ABI tests under the clang
sanitizer runtime (tests/test_sanitized_abi.py).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libsparse_attn.so")
# measurement context only (bench.py): a matrix-pipe throughput probe
PROBE_SRC = os.path.join(CSRC, "probe", "mfma_probe.hip")
PROBE_LIB = os.path.join(LIB_DIR, "libsa_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # no packed-fp32 instruction selection in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# host-only instrumentation: each sanitizer flag applies to the host pass only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_OBJ = os.path.join(OBJ, "san")
SAN_LIB = os.path.join(SAN_OBJ, "libsparse_attn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def sanitizer_runtime() -> str:
    """clang's shared AddressSanitizer runtime (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under " + ROCM)
    return hits[-1]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OBJ if sanitize else OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + (HOST_SANITIZE if sanitize else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build_sanitized(verbose: bool = True) -> str:
    """The host-instrumented library (see the module docstring)."""
    os.makedirs(SAN_OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize=True), srcs))
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    cmd = [clangxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
           "-o", SAN_LIB] + objs + ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                                   "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = True) -> str:
    """libsa_probe.so: the matrix-pipe probe bench.py reports as context."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
