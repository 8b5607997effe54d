"""Build libkda.so (the gfx950 HIP kernels plus the C ABI) in-tree with hipcc.

    python -m gated_delta_rule_39_amd.build [--asan | --phases]

writes gated_delta_rule_39_amd/_lib/libkda.so.  Every translation unit is compiled
for gfx950 only, with packed-fp32 instruction selection disabled.  --asan writes a
copy to _lib/asan/libkda.so whose host code (the C ABI, argument checks, plans,
launches) is built with AddressSanitizer; the device code is the same.  It needs the
sanitizer runtime preloaded into the loading process (tests/test_abi_asan.py).
--phases writes a timing build to _lib/phase/libkda.so: the same kernels with
-DKDA_PHASE_STAMPS, whose producer/consumer workgroups record per-phase s_memtime
sums (read by `bench.py --phases`).  The product library never contains them.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libkda.so")

SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_backward.hip",
           "kda_probe.hip", "kda_noalloc.hip"]
ARCH = "gfx950"
# -packed-fp32-ops: no v_pk_*_f32 generation.  -amdgpu-mfma-vgpr-form: MFMA
# accumulators in ordinary VGPRs, so loop-carried accumulators (the prefill state)
# are scaled and packed in place instead of being copied out of and back into AGPRs.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the KDA library needs the ROCm toolchain to build")


# host code only: each -fsanitize= right after -Xarch_host
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(hipcc: str, src: str, obj: str, verbose: bool, extra=()):
    lang = ["-x", "hip"]
    cmd = [hipcc, *lang, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


ASAN_LIB = os.path.join(OUT_DIR, "asan", "libkda.so")
PHASE_LIB = os.path.join(OUT_DIR, "phase", "libkda.so")


def build(verbose: bool = False, asan: bool = False, phases: bool = False) -> str:
    """Compile every source and link libkda.so (asan: the host-sanitized copy;
    phases: the timing build with phase stamps); returns the library path."""
    if asan and phases:
        raise ValueError("one variant at a time")
    hipcc = _hipcc()
    lib = ASAN_LIB if asan else PHASE_LIB if phases else LIB
    extra = ASAN_FLAGS if asan else ["-DKDA_PHASE_STAMPS"] if phases else []
    obj_dir = os.path.join(os.path.dirname(lib), "obj")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(hipcc, so[0], so[1], verbose, extra), zip(SOURCES, objs)))
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libkda.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv,
                phases="--phases" in sys.argv))
