"""Build libmsr.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m retnet_scale_retention_amd.build [jobs] [--sanitize]
Every source is compiled for gfx950 only; objects go to _build/, the shared
library to retnet_scale_retention_amd/libmsr.so.  --sanitize builds
libmsr_asan.so instead (objects in _build_asan/): the host code (argument
validation, workspace plans, launch set-up) with AddressSanitizer and
UndefinedBehaviorSanitizer, the device code unchanged.  It runs on the CPU
with clang's ASan runtime preloaded (tests/test_sanitized_cpu.py).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libmsr.so"
BUILD = PKG / "_build"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# packed-fp32 instructions are disabled for all device code
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# MFMA accumulators in architectural VGPRs where they fit: with accumulators
# in AGPRs the register allocator chains copies between them around loops,
# which serialises the matrix pipe (a 16x16x32 bf16 MFMA loop with one wave
# per SIMD then issues every ~31 clocks instead of ~19)
MFMA_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
MFMA_SOURCES = {"k_chunk_mfma.hip", "k_proj.hip"}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{ROOT / 'include'}", f"-I{CSRC}"]
# host-side sanitizers only (each flag bound to the host pass)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
ASAN_OUT = PKG / "libmsr_asan.so"
ASAN_BUILD = PKG / "_build_asan"


def sources():
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def _compile(src: Path, sanitize: bool = False) -> Path:
    obj = (ASAN_BUILD if sanitize else BUILD) / (src.name + ".o")
    extra = MFMA_FLAGS if src.name in MFMA_SOURCES else []
    san = SANITIZE if sanitize else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, *san, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd = [HIPCC, *COMMON, *san, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{r.stderr}")
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> Path:
    bdir, out = (ASAN_BUILD, ASAN_OUT) if sanitize else (BUILD, OUT)
    bdir.mkdir(exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    tmp = out.with_suffix(".so.tmp")
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    print(build(int(args[0]) if args else 8, sanitize="--sanitize" in sys.argv))
