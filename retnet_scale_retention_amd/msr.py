"""Thin ctypes binding of libmsr.so (include/msr.h).

Argument marshalling only: every step of the operation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
If libmsr.so is missing this module raises on first use -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import numpy as np

import os

LIB_PATH = Path(os.environ.get("MSR_LIB", Path(__file__).resolve().parent / "libmsr.so"))

MSR_OK = 0
MSR_F32, MSR_BF16 = 0, 1
MSR_FLAG_NO_ROTATE, MSR_FLAG_NO_GROUPNORM, MSR_FLAG_DECAY_ROWNORM, MSR_FLAG_SPLIT_SCORES, MSR_FLAG_FUSED = 1, 2, 4, 8, 16
MSR_EXCHANGE_AUTO, MSR_EXCHANGE_OFF, MSR_EXCHANGE_NO_WAIT = 0, 1, 2
MSR_FORM_PARALLEL, MSR_FORM_CHUNKWISE, MSR_FORM_STEP, MSR_FORM_BACKWARD, MSR_FORM_QKV_CHUNKWISE = 0, 1, 2, 3, 4
STATUS = {0: "MSR_OK", -1: "MSR_ERR_INVALID_ARG", -2: "MSR_ERR_SHAPE", -3: "MSR_ERR_DTYPE",
          -4: "MSR_ERR_UNSUPPORTED", -5: "MSR_ERR_WORKSPACE", -6: "MSR_ERR_HIP"}

EXPORTS = ("msr_abi_version", "msr_last_error", "msr_workspace_size", "msr_workspace_bytes", "msr_parallel",
           "msr_chunkwise", "msr_chunkwise_noalloc", "msr_chunkwise_backward", "msr_qkv_projection", "msr_qkv_chunkwise",
           "msr_recurrent_step", "msr_set_kernel_events", "msr_set_exchange")


class MsrError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {what}")


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("gamma", ctypes.POINTER(ctypes.c_float)), ("theta", ctypes.POINTER(ctypes.c_float)),
        ("scale", ctypes.c_float), ("gn_eps", ctypes.c_float),
        ("pos0", ctypes.c_int64), ("flags", ctypes.c_uint32),
        ("pos_rows", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load libmsr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m retnet_scale_retention_amd.build`")
    lib = ctypes.CDLL(str(LIB_PATH))
    P = ctypes.POINTER(Problem)
    vp, fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
    lib.msr_abi_version.argtypes, lib.msr_abi_version.restype = [], ctypes.c_int
    lib.msr_last_error.argtypes, lib.msr_last_error.restype = [], ctypes.c_char_p
    lib.msr_workspace_size.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.msr_workspace_size.restype = ctypes.c_int
    lib.msr_workspace_bytes.argtypes = [P, ctypes.c_int32, ctypes.c_int32]
    lib.msr_workspace_bytes.restype = ctypes.c_size_t
    lib.msr_parallel.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msr_parallel.restype = ctypes.c_int
    lib.msr_chunkwise.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msr_chunkwise.restype = ctypes.c_int
    lib.msr_chunkwise_noalloc.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp]
    lib.msr_chunkwise_noalloc.restype = ctypes.c_int
    lib.msr_chunkwise_backward.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_size_t, vp]
    lib.msr_chunkwise_backward.restype = ctypes.c_int
    lib.msr_qkv_projection.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.msr_qkv_projection.restype = ctypes.c_int
    lib.msr_qkv_chunkwise.argtypes = [P, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.msr_qkv_chunkwise.restype = ctypes.c_int
    lib.msr_recurrent_step.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.msr_recurrent_step.restype = ctypes.c_int
    lib.msr_set_kernel_events.argtypes = [vp, vp]
    lib.msr_set_kernel_events.restype = None
    lib.msr_set_exchange.argtypes, lib.msr_set_exchange.restype = [ctypes.c_int32], ctypes.c_int
    del fp
    _lib = lib
    return lib


def _check(status: int):
    if status != MSR_OK:
        raise MsrError(status, load().msr_last_error().decode(errors="replace"))


class _Desc:
    """A Problem plus the host arrays it points to (kept alive)."""

    def __init__(self, B, T, H, dk, dv, dtype, gamma, theta=None, scale=0.0, eps=1e-5, pos0=0, flags=0,
                 pos_rows=None):
        self.gamma = np.ascontiguousarray(gamma, dtype=np.float32)
        if self.gamma.shape != (H,):
            raise ValueError(f"gamma must hold H={H} values")
        self.theta = None if theta is None else np.ascontiguousarray(theta, dtype=np.float32)
        if self.theta is not None and self.theta.shape != (dk // 2,):
            raise ValueError(f"theta must hold dk/2={dk // 2} values")
        fptr = lambda a: (ctypes.POINTER(ctypes.c_float)() if a is None
                          else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        self.p = Problem(B, T, H, dk, dv, dtype, fptr(self.gamma), fptr(self.theta),
                         float(scale), float(eps), int(pos0), int(flags), pos_rows)

    @property
    def ref(self):
        return ctypes.byref(self.p)


def workspace_size(B, T, H, dk, dv, dtype, gamma, form, chunk=0, **kw) -> int:
    d = _Desc(B, T, H, dk, dv, dtype, gamma, **kw)
    n = ctypes.c_size_t(0)
    _check(load().msr_workspace_size(d.ref, form, chunk, ctypes.byref(n)))
    return int(n.value)


# --------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return MSR_F32
    if t.dtype == torch.bfloat16:
        return MSR_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    torch = _torch()
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _prep(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B, T, H, dk] and v [B, T, H, dv]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    return (*q.shape, v.shape[3])


def _pos_rows(pos_rows, B, device):
    """Device address of a per-batch-row position tensor (int64 [B]), or None."""
    torch = _torch()
    if pos_rows is None:
        return None
    if (pos_rows.dtype != torch.int64 or tuple(pos_rows.shape) != (B,) or not pos_rows.is_contiguous()
            or pos_rows.device != device):
        raise ValueError(f"pos_rows must be a contiguous int64 [B={B}] tensor on {device}")
    return pos_rows.data_ptr()


def _form(fn, form, q, k, v, gamma, chunk, theta, scale, eps, pos0, flags, state_in,
          return_state, out, state_out, workspace, stream, pos_rows=None):
    torch = _torch()
    B, T, H, dk, dv = _prep(q, k, v)
    code = _dtype_code(q)
    d = _Desc(B, T, H, dk, dv, code, gamma, theta, scale, eps, pos0, flags, _pos_rows(pos_rows, B, q.device))
    n = ctypes.c_size_t(0)
    _check(load().msr_workspace_size(d.ref, form, chunk, ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if state_in is not None and (state_in.dtype != torch.float32 or not state_in.is_contiguous()
                                 or tuple(state_in.shape) != (B, H, dk, dv)):
        raise ValueError("state_in must be a contiguous float32 [B, H, dk, dv] tensor")
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    args = [d.ref]
    if form == MSR_FORM_CHUNKWISE:
        args.append(int(chunk))
    args += [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_in), _ptr(state_out),
             _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(q, stream)]
    _check(fn(*args))
    return out, state_out


def msr_parallel(q, k, v, gamma, *, theta=None, scale=0.0, eps=1e-5, pos0=0, flags=0,
                 state_in=None, return_state=True, out=None, state_out=None, workspace=None,
                 stream=None, pos_rows=None):
    """Parallel form. q, k: [B, T, H, dk]; v: [B, T, H, dv] (float32 or bfloat16,
    on the device); gamma: H host values; pos_rows: optional int64 [B] device
    tensor of per-row start positions (else every row starts at pos0).
    Returns (O, state_out or None)."""
    return _form(load().msr_parallel, MSR_FORM_PARALLEL, q, k, v, gamma, 0, theta, scale, eps,
                 pos0, flags, state_in, return_state, out, state_out, workspace, stream, pos_rows)


def msr_chunkwise(q, k, v, gamma, chunk, *, theta=None, scale=0.0, eps=1e-5, pos0=0, flags=0,
                  state_in=None, return_state=True, out=None, state_out=None, workspace=None,
                  stream=None, pos_rows=None):
    """Chunkwise-recurrent form with chunk size `chunk` (a last chunk shorter
    than `chunk` takes the remaining tokens when chunk does not divide T)."""
    return _form(load().msr_chunkwise, MSR_FORM_CHUNKWISE, q, k, v, gamma, chunk, theta, scale,
                 eps, pos0, flags, state_in, return_state, out, state_out, workspace, stream, pos_rows)


NOALLOC_SCRATCH_BYTES = 64 << 20  # MSR_NOALLOC_SCRATCH_BYTES


def msr_chunkwise_noalloc(q, k, v, gamma, chunk, *, out, state_out=None, theta=None, scale=0.0, eps=1e-5, pos0=0,
                          flags=0, state_in=None, stream=None, pos_rows=None):
    """msr_chunkwise with the library's fixed per-GPU scratch array instead of
    a workspace: allocates nothing (out and state_out are the caller's).
    Returns (O, state_out)."""
    torch = _torch()
    B, T, H, dk, dv = _prep(q, k, v)
    d = _Desc(B, T, H, dk, dv, _dtype_code(q), gamma, theta, scale, eps, pos0, flags,
              _pos_rows(pos_rows, B, q.device))
    if tuple(out.shape) != (B, T, H, dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, T, H, dv] tensor of q's dtype")
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, dk, dv)):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, dk, dv] tensor")
    _check(load().msr_chunkwise_noalloc(d.ref, int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_in),
                                        _ptr(state_out), _stream(q, stream)))
    return out, state_out


def msr_chunkwise_backward(q, k, v, gamma, chunk, grad_out, *, grad_state=None, state_in=None, theta=None,
                           scale=0.0, eps=1e-5, pos0=0, flags=0, pos_rows=None, want_state_grad=True,
                           workspace=None, stream=None):
    """Gradients of the chunkwise (= parallel) form through rotation, scale,
    retention and GroupNorm.  grad_out: dL/dO [B, T, H, dv] (dtype of q);
    grad_state: dL/dstate_out [B, H, dk, dv] float32 or None.  Returns
    (dQ, dK, dV, dstate_in or None), dQ/dK/dV in the dtype of q."""
    torch = _torch()
    B, T, H, dk, dv = _prep(q, k, v)
    if tuple(grad_out.shape) != (B, T, H, dv) or grad_out.dtype != q.dtype or not grad_out.is_contiguous():
        raise ValueError("grad_out must be a contiguous [B, T, H, dv] tensor of q's dtype")
    for name, t in (("state_in", state_in), ("grad_state", grad_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, dk, dv)):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, dk, dv] tensor")
    d = _Desc(B, T, H, dk, dv, _dtype_code(q), gamma, theta, scale, eps, pos0, flags,
              _pos_rows(pos_rows, B, q.device))
    n = ctypes.c_size_t(0)
    _check(load().msr_workspace_size(d.ref, MSR_FORM_BACKWARD, chunk, ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if want_state_grad else None
    _check(load().msr_chunkwise_backward(d.ref, int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(state_in),
                                         _ptr(grad_out), _ptr(grad_state), _ptr(dq), _ptr(dk_), _ptr(dv_),
                                         _ptr(ds), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                         _stream(q, stream)))
    return dq, dk_, dv_, ds


def _qkv_args(x, wq, wk, wv, H):
    for name, t in (("x", x), ("wq", wq), ("wk", wk), ("wv", wv)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if x.dim() != 3 or wq.dim() != 2 or wk.shape != wq.shape or wv.dim() != 2:
        raise ValueError("expected x [B, T, d_model], wq, wk [H dk, d_model], wv [H dv, d_model]")
    B, T, dm = x.shape
    if wq.shape[1] != dm or wv.shape[1] != dm or wq.shape[0] % H or wv.shape[0] % H:
        raise ValueError("weight shapes do not match d_model and H")
    return B, T, dm, wq.shape[0] // H, wv.shape[0] // H


def msr_qkv_projection(x, wq, wk, wv, H, *, theta=None, scale=0.0, pos0=0, flags=0, pos_rows=None,
                       out=None, stream=None):
    """Q = R(x wq^T), K = s R(x wk^T), V = x wv^T as [B, T, H, d] bf16
    (x [B, T, d_model] bf16, weights [H d, d_model]).  Returns (Q, K, V)."""
    torch = _torch()
    B, T, dm, dk, dv = _qkv_args(x, wq, wk, wv, H)
    d = _Desc(B, T, H, dk, dv, _dtype_code(x), np.ones(H, np.float32), theta, scale, 1e-5, pos0, flags,
              _pos_rows(pos_rows, B, x.device))
    if out is None:
        out = (torch.empty((B, T, H, dk), dtype=x.dtype, device=x.device),
               torch.empty((B, T, H, dk), dtype=x.dtype, device=x.device),
               torch.empty((B, T, H, dv), dtype=x.dtype, device=x.device))
    _check(load().msr_qkv_projection(d.ref, int(dm), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv),
                                     *(_ptr(t) for t in out), _stream(x, stream)))
    return out


def msr_qkv_chunkwise(x, wq, wk, wv, gamma, chunk, *, theta=None, scale=0.0, eps=1e-5, pos0=0, flags=0,
                      state_in=None, return_state=True, out=None, state_out=None, workspace=None,
                      stream=None, pos_rows=None):
    """The projections followed by the chunkwise form: returns (O, state_out
    or None) for the layer input x [B, T, d_model] and weights [H d, d_model]."""
    torch = _torch()
    H = len(np.atleast_1d(gamma))
    B, T, dm, dk, dv = _qkv_args(x, wq, wk, wv, H)
    d = _Desc(B, T, H, dk, dv, _dtype_code(x), gamma, theta, scale, eps, pos0, flags,
              _pos_rows(pos_rows, B, x.device))
    n = ctypes.c_size_t(0)
    _check(load().msr_workspace_size(d.ref, MSR_FORM_QKV_CHUNKWISE, chunk, ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=x.dtype, device=x.device)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=x.device)
    _check(load().msr_qkv_chunkwise(d.ref, int(chunk), int(dm), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv),
                                    _ptr(out), _ptr(state_in), _ptr(state_out), _ptr(workspace),
                                    ctypes.c_size_t(workspace.numel()), _stream(x, stream)))
    return out, state_out


def msr_recurrent_step(q, k, v, state, gamma, pos, *, theta=None, scale=0.0, eps=1e-5, flags=0,
                       out=None, stream=None):
    """One decode step at absolute position `pos` (an int, or an int64 [B]
    device tensor with one position per batch row); q, k: [B, H, dk],
    v: [B, H, dv]; state [B, H, dk, dv] float32 is updated in place.
    Returns o [B, H, dv]."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("state", state)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, H, dk = q.shape
    dv = v.shape[2]
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv):
        raise ValueError("state must be float32 [B, H, dk, dv]")
    if isinstance(pos, torch.Tensor):
        d = _Desc(B, 1, H, dk, dv, _dtype_code(q), gamma, theta, scale, eps, 0, flags,
                  _pos_rows(pos, B, q.device))
    else:
        d = _Desc(B, 1, H, dk, dv, _dtype_code(q), gamma, theta, scale, eps, pos, flags)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _check(load().msr_recurrent_step(d.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state),
                                     _stream(q, stream)))
    return out


def set_kernel_events(start=None, stop=None):
    """Measurement hook: record the hipEvent handles `start` / `stop` (ints
    or None) around the main kernel of every later call on this thread."""
    load().msr_set_kernel_events(ctypes.c_void_p(start) if start else None,
                                 ctypes.c_void_p(stop) if stop else None)


def set_exchange(mode: int):
    """Process-wide GroupNorm finishing of the split-row chunk kernel
    (MSR_EXCHANGE_AUTO, MSR_EXCHANGE_OFF or MSR_EXCHANGE_NO_WAIT; include/msr.h)."""
    _check(load().msr_set_exchange(int(mode)))
