"""Builds libnosa.so (the C-ABI HIP library) in-tree for gfx950.

Each .hip file under csrc/ is compiled with hipcc; the objects are linked
against the HIP runtime that PyTorch ships, found by name
(``libamdhip64.so``), so a process that has imported torch uses exactly one
HIP runtime for torch's memory and for these kernels.

Usage: python -m trainable_offloadable_block_amd.build  (or build());
``--phase-clocks`` builds the timing variant libnosa_clocks.so instead.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libnosa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=fast",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required")
    return path


def _torch_lib_dir() -> str:
    import torch
    d = os.path.join(os.path.dirname(torch.__file__), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so in {d}")
    return d


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip"))


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE,
           "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = [ln for ln in r.stderr.splitlines() if ln.strip() and noise not in ln]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(verbose: bool = True, out_path: str = LIB_PATH, defines=()) -> str:
    """Compiles every HIP source and links libnosa.so (or out_path, with
    extra preprocessor defines for a tuning variant); returns its path."""
    build_dir = BUILD_DIR if out_path == LIB_PATH else out_path + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), srcs))
    tlib = _torch_lib_dir()
    tmp = out_path + ".tmp"
    cmd = ["g++", "-shared", "-o", tmp, *objs, f"-L{tlib}", "-lamdhip64",
           f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined", "-lstdc++"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out_path)
    if verbose:
        print(f"built {out_path}")
    return out_path


CLOCKS_LIB_PATH = os.path.join(PKG, "libnosa_clocks.so")


def build_phase_clocks(verbose: bool = True) -> str:
    """The timing build: the same library with phase clocks in the append +
    select and decode kernels (NOSA_PHASE_CLOCKS), as libnosa_clocks.so. Load
    it with NOSA_LIBRARY=<path> (bench.py --phase-clocks)."""
    return build(verbose, CLOCKS_LIB_PATH, defines=("NOSA_PHASE_CLOCKS",))


if __name__ == "__main__":
    if "--phase-clocks" in sys.argv[1:]:
        build_phase_clocks()
    else:
        build()
