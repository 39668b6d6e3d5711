"""Build libpda.so (the C-ABI library with its gfx950 kernels) in-tree.

    python -m paged_split_decode_amd.build

Each .hip source compiles to an object in parallel; the objects link into
paged_split_decode_amd/libpda.so. Packed-fp32 instruction selection is turned
off for the device code (-packed-fp32-ops); the host pass warns that it does
not know that feature, which is harmless.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpda.so")
ARCH = "gfx950"

SOURCES = ["pda_api.hip", "pda_combine.hip", "pda_decode_f16.hip",
           "pda_decode_fp8.hip", "pda_decode_i8.hip", "pda_writer.hip", "pda_prefill.hip",
           "pda_noalloc.hip", "pda_probe.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


# Per-source flags. The prefill kernel's staged K/V are finite by construction
# (slots past a sequence are zeroed), so its max operations need no NaN
# canonicalization. The attention kernels take the VGPR form of the MFMA
# instructions: at one wave per SIMD the compiler otherwise keeps the score and
# output accumulators in AGPRs and copies all of them to VGPRs on every page,
# for a rescale that is rarely taken (AGPRs remain in use as spill space).
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"pda_prefill.hip": ["-fno-honor-nans", *_VGPR_MFMA], "pda_decode_f16.hip": _VGPR_MFMA,
         "pda_decode_fp8.hip": _VGPR_MFMA, "pda_decode_i8.hip": _VGPR_MFMA}


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False, defines: tuple = (), lib: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link `lib`. `defines` (-D flags) and another
    `lib` / `build_dir` make a diagnostic variant beside the library."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, tuple(defines)), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
