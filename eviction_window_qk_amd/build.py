"""Build libkvc.so (the HIP library behind include/kvc.h) in-tree for gfx950.

    python -m eviction_window_qk_amd.build          # compile + link
    python -m eviction_window_qk_amd.build --check  # also run nm on the exports

Every source compiles with hipcc for --offload-arch=gfx950.  Packed fp32
instructions are disabled for all device code; the mass/segmentation unit
additionally compiles with -ffp-contract=off (its integer decisions follow an
exact one-operation-at-a-time contract).  Objects go to _build/, the shared
library lands next to this file, replaced atomically.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = {
    "kvc_host.cpp": [],
    "kvc_score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],  # MFMA accumulators in VGPRs: no copies for the softmax VALU work
    "kvc_mass.hip": ["-ffp-contract=off"],
    "kvc_select.hip": [],
    "kvc_gather.hip": [],
    "kvc_refresh.hip": ["-ffp-contract=off"],  # fp64 cosine: one operation at a time
    "kvc_noalloc.hip": [],
}
EXPORTS = ["kvc_score_window", "kvc_mass_segment", "kvc_select", "kvc_gather_compact",
           "kvc_gather_paged", "kvc_qc_trigger", "kvc_partial_init", "kvc_partial_append",
           "kvc_full_sync", "kvc_compress_event", "kvc_compress_event_noalloc",
           "kvc_workspace_bytes", "kvc_segment_capacity",
           "kvc_check_params", "kvc_strerror", "kvc_abi_version"]


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *lang, *DEVICE, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln]           # host pass warns about the device flag
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(errs))
    if errs:
        print(f"[build] {src}:\n" + "\n".join(errs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        futs = {src: ex.submit(_compile, src, extra) for src, extra in SOURCES.items()}
        objs = [futs[src].result() for src in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB}")
    return LIB


def exported_symbols(lib: str = LIB) -> set:
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    out = subprocess.run([nm, "-D", "--defined-only", lib], capture_output=True, text=True).stdout
    return {ln.split()[-1] for ln in out.splitlines() if ln.strip()}


if __name__ == "__main__":
    build()
    if "--check" in sys.argv:
        missing = [s for s in EXPORTS if s not in exported_symbols()]
        if missing:
            sys.exit(f"missing exports: {missing}")
        print("[build] all exports present")
