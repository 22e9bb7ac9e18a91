"""fp64 CPU oracle for multi-scale retention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It wraps ``oracle.c`` (plain loops in
double precision, OpenMP over independent (batch, head) pairs) through ctypes
and shares nothing with the HIP library: no code, header, table or constant.

Inputs are the exact values handed to the GPU (fp32, or bf16 values held in
fp32), promoted to fp64.  Parameters the GPU receives as fp32 (gamma, theta,
scale, eps) are used here as the same fp32 values, promoted.

Page references (by site and section):
  jsqmd.com "From RoPE to Retention" -- s2 theta_shift rotation, s3 decay
      mask and per-head gamma, s4.1/4.2/4.3 the three forms, s5 GroupNorm and
      the 1/sqrt(d) scale, zero initial state.
  aiqz.cc RetNet tutorial -- decay mask, parallel / recurrent / chunkwise
      representations, the numpy demo of parallel-vs-recurrent agreement.
  b99b.cn QbitAI article -- the three forms, GroupNorm's scale invariance.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
# MSR_ORACLE_LIB selects another build of oracle.c (the sanitized one of
# tests/test_sanitized_cpu.py); the default is the gcc build below
_LIB = Path(os.environ.get("MSR_ORACLE_LIB", _HERE / "liboracle.so"))
_ASAN_LIB = _HERE / "liboracle_asan.so"
_lib = None


def build(force: bool = True, sanitize: bool = False) -> Path:
    """Compile oracle.c with gcc (IEEE arithmetic: no fast-math).  With
    sanitize: with clang and AddressSanitizer + UndefinedBehaviorSanitizer
    into liboracle_asan.so (the runtime clang's hipcc builds use too)."""
    lib = _ASAN_LIB if sanitize else _LIB
    if force or not lib.exists() or lib.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = lib.with_suffix(".so.tmp")
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                   "-fno-omit-frame-pointer", str(_SRC), "-o", str(tmp), "-lm"]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                   str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
        ("dk", ctypes.c_int), ("dv", ctypes.c_int),
        ("gamma", ctypes.POINTER(ctypes.c_double)),
        ("theta", ctypes.POINTER(ctypes.c_double)),
        ("scale", ctypes.c_double), ("eps", ctypes.c_double),
        ("pos0", ctypes.c_int64), ("rotate", ctypes.c_int), ("groupnorm", ctypes.c_int),
        ("rownorm", ctypes.c_int),
    ]


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=False)
        lib = ctypes.CDLL(str(_LIB))
        dp = ctypes.POINTER(ctypes.c_double)
        pp = ctypes.POINTER(_Problem)
        for name in ("oracle_parallel", "oracle_recurrent"):
            f = getattr(lib, name)
            f.argtypes = [pp, dp, dp, dp, dp, dp, dp]
            f.restype = ctypes.c_int
        lib.oracle_chunkwise.argtypes = [pp, ctypes.c_int, dp, dp, dp, dp, dp, dp]
        lib.oracle_chunkwise.restype = ctypes.c_int
        lib.oracle_parallel_rows.argtypes = [pp, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                             dp, dp, dp, dp, dp]
        lib.oracle_parallel_rows.restype = ctypes.c_int
        lib.oracle_rotate.argtypes = [pp, dp, ctypes.c_double, dp]
        lib.oracle_rotate.restype = None
        lib.oracle_groupnorm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, dp]
        lib.oracle_groupnorm.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_theta(dk: int) -> np.ndarray:
    """theta_i = 10000^(-2i/d_k) for pair i, evaluated in fp64 and held as
    fp32 (the precision of the theta parameter)."""
    i = np.arange(dk // 2, dtype=np.float64)
    return (10000.0 ** (-2.0 * i / dk)).astype(np.float32)


def default_scale(dk: int) -> float:
    """d_k^-0.5, held as fp32 like the scale parameter."""
    return float(np.float32(1.0 / np.sqrt(np.float64(dk))))


class _Call:
    """Marshals one problem description; keeps the fp64 buffers alive."""

    def __init__(self, shape_q, dv, gamma, theta, scale, eps, pos0, rotate, groupnorm, rownorm=False):
        B, T, H, dk = shape_q
        self.gamma = _f64(np.asarray(gamma, dtype=np.float32))
        if self.gamma.shape != (H,):
            raise ValueError("gamma must have one value per head")
        th = default_theta(dk) if theta is None else np.asarray(theta, dtype=np.float32)
        self.theta = _f64(th)
        sc = default_scale(dk) if scale is None else float(np.float32(scale))
        self.p = _Problem(B, T, H, dk, dv, _ptr(self.gamma), _ptr(self.theta), sc,
                          float(np.float32(eps)), int(pos0), int(bool(rotate)),
                          int(bool(groupnorm)), int(bool(rownorm)))


def _run(fn, q, k, v, gamma, *, chunk=None, theta=None, scale=None, eps=1e-5, pos0=0,
         rotate=True, groupnorm=True, rownorm=False, s_in=None, outputs=True, state=True):
    q, k, v, s_in = _f64(q), _f64(k), _f64(v), _f64(s_in)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, H):
        raise ValueError("q, k, v shapes disagree")
    if s_in is not None and s_in.shape != (B, H, dk, dv):
        raise ValueError("state shape must be [B, H, dk, dv]")
    c = _Call(q.shape, dv, gamma, theta, scale, eps, pos0, rotate, groupnorm, rownorm)
    o = np.zeros((B, T, H, dv)) if outputs else None
    s_out = np.zeros((B, H, dk, dv)) if state else None
    lib = _load()
    args = [ctypes.byref(c.p)]
    if chunk is not None:
        args.append(int(chunk))
    args += [_ptr(q), _ptr(k), _ptr(v), _ptr(s_in), _ptr(o), _ptr(s_out)]
    rc = getattr(lib, fn)(*args)
    if rc != 0:
        raise ValueError(f"{fn} failed with code {rc}")
    return o, s_out


def parallel(q, k, v, gamma, **kw):
    """Parallel form (the plain definition).  Returns (O, S_out)."""
    return _run("oracle_parallel", q, k, v, gamma, **kw)


def recurrent(q, k, v, gamma, **kw):
    """Recurrent form, one token at a time.  Returns (O, S_out)."""
    return _run("oracle_recurrent", q, k, v, gamma, **kw)


def chunkwise(q, k, v, gamma, chunk, **kw):
    """Chunkwise-recurrent form with chunk size `chunk`.  Returns (O, S_out)."""
    return _run("oracle_chunkwise", q, k, v, gamma, chunk=chunk, **kw)


def step(q, k, v, state, gamma, pos, **kw):
    """One recurrent decode step at absolute position `pos`.
    q, k: [B, H, dk]; v: [B, H, dv]; state: [B, H, dk, dv].
    Returns (o [B, H, dv], new state)."""
    q4, k4, v4 = (np.asarray(x)[:, None] for x in (q, k, v))
    o, s = recurrent(q4, k4, v4, gamma, s_in=state, pos0=pos, **kw)
    return o[:, 0], s


def parallel_rows(q, k, v, gamma, rows, *, theta=None, scale=None, eps=1e-5, pos0=0,
                  rotate=True, groupnorm=True, rownorm=False, s_in=None):
    """Selected rows of the parallel definition for ONE (batch, head) pair.
    q, k: [T, dk]; v: [T, dv]; gamma: scalar; s_in: [dk, dv] or None.
    Returns [len(rows), dv]."""
    q, k, v, s_in = _f64(q), _f64(k), _f64(v), _f64(s_in)
    T, dk = q.shape
    dv = v.shape[1]
    c = _Call((1, T, 1, dk), dv, [gamma], theta, scale, eps, pos0, rotate, groupnorm, rownorm)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(r), dv))
    rc = _load().oracle_parallel_rows(ctypes.byref(c.p), len(r),
                                      r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(s_in), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_parallel_rows failed with code {rc}")
    return out


def rotate(x, *, theta=None, pos0=0, factor=1.0):
    """theta_shift of a [B, T, H, dk] tensor at positions pos0 + t, times factor."""
    x = _f64(x)
    B, T, H, dk = x.shape
    c = _Call(x.shape, 1, np.ones(H, np.float32), theta, 1.0, 1e-5, pos0, True, False)
    y = np.zeros_like(x)
    _load().oracle_rotate(ctypes.byref(c.p), _ptr(x), float(factor), _ptr(y))
    return y


def project(x, w):
    """A linear layer without bias, x [..., d_model] times w [out, d_model]
    transposed, in fp64: the projections that give Q, K and V from the
    layer input (jsqmd.com s2)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def groupnorm(x, eps=1e-5):
    """GroupNorm over the last axis of x (one group per row), no affine."""
    x = _f64(x).copy()
    n = x.shape[-1]
    _load().oracle_groupnorm(int(x.size // n), int(n), float(np.float32(eps)), _ptr(x))
    return x
