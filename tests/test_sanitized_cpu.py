"""The CPU suite again under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host code of libmsr (argument validation, workspace plans, launch
set-up; the device code is unchanged) and the fp64 oracle with both
sanitizers, then runs the ABI checks and the oracle pins in a child Python
with clang's ASan runtime preloaded.  Any invalid access or undefined
behaviour aborts the child and fails this test.  CPU only."""
import glob
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SUITES = ["tests/test_abi_cpu.py", "tests/test_oracle_pins.py", "tests/test_oracle_grad_pins.py"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def stale(out, srcs):
    return not out.exists() or any(s.stat().st_mtime > out.stat().st_mtime for s in srcs)


def test_cpu_suite_under_asan_and_ubsan():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    from oracle import oracle
    from retnet_scale_retention_amd import build as b
    lib = b.ASAN_OUT
    if stale(lib, b.sources() + sorted(b.CSRC.glob("*.hpp")) + [ROOT / "include" / "msr.h"]):
        b.build(sanitize=True)
    olib = oracle.build(force=False, sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, MSR_LIB=str(lib), MSR_ORACLE_LIB=str(olib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
