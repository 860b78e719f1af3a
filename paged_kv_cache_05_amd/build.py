"""Build libpa.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_kv_cache_05_amd.build        # or: from paged_kv_cache_05_amd.build import build

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in parallel), then linked
into ``paged_kv_cache_05_amd/libpa.so``.  Packed-fp32 instructions are disabled for all device
code (``-packed-fp32-ops``).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libpa.so"
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source compiler options.  The 16-bit matrix-core decode keeps its MFMA accumulators in
# ordinary VGPRs: left to its heuristics the compiler put them in AGPRs (about 250 registers,
# two waves per SIMD) and copied all 32 of them into VGPRs on every chunk for the rarely taken
# rescale.  The 256-dim instances keep the compiler's choice: their 16 KiB chunks and 64
# accumulators need more than the 256 VGPRs one wave can address.
EXTRA_FLAGS = {
    "pa_decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "pa_decode_mfma_d64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "pa_decode_mfma_d80.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def sources():
    return sorted(CSRC.glob("*.hip"))


def _compile(src: pathlib.Path, verbose: bool) -> pathlib.Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src.name, []), "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> pathlib.Path:
    """Compile every HIP source and link libpa.so; always rebuilds."""
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
