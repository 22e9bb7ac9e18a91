#!/usr/bin/env python3
"""Benchmark of the multi-scale retention hot path on one MI355X.

One "step" is one chunkwise forward (rotation prologue, intra-chunk MFMA
products, decay mask, cross-chunk term, state carry, GroupNorm) over the
7B-shaped layer: B=2, T=8192, H=16, d_k=256, d_v=512, chunk 128, bf16 in,
fp32 state.  `value` is that forward's throughput in tokens/s with inputs
already resident in HBM.  The same JSON line also reports
  - roofline: the chunk-recurrence kernel alone (the dominant kernel, which
    also normalises the rows when they span 2-8 of its slices), timed
    with HIP events recorded around it on its own stream (library measurement
    hook), against the bf16 dense MFMA peak, with its algorithmic flops
    4 d_k d_v (inter-chunk term and state update) + (b+1) d_v (causal value
    product) per token and head; the scores (b+1) d_k run in the prep kernel.
    step_tflops counts F = (b+1)(d_k+d_v) + 4 d_k d_v per token and head over
    the whole call;
  - decode: the recurrent decode step at B=64, H=16, d_k=256, d_v=512 after a
    2048-token chunkwise prefill, 1024 steps, against the HBM peak;
  - parallel: the parallel form over the same 7B-shaped layer (O(T^2) score
    blocks, one call), algorithmic flops (T+1)(d_k+d_v) + 4 d_k d_v per token
    and head;
  - backward: msr_chunkwise_backward on the small and the 7B-shaped layers;
  - qkv: the Q/K/V projections (d_model = 4096) with the rotation in the
    GEMM epilogue, and the projections + chunkwise form together;
  - other_chunk: the same forward at the workload's other chunk size (256);
  - fused_schedule: the same forward with MSR_FLAG_FUSED (rotation, scores and
    GroupNorm inside the recurrence workgroups; fewer HBM bytes, not the
    default), here and at the long sequence's chunks 64 and 128;
  - long_sequence: the chunkwise forward over B=1, T=131072, H=8, d_k=128,
    d_v=256 at chunk 64, 128 and 256 (state carried across all chunks);
  - cpu_baseline: the fp64 oracle's chunkwise form timed on a bounded sample
    of the same workload on the host cores (a reported baseline only);
  - achievable_peaks: a 1 GiB device copy and a bf16 8192^3 matrix product
    through torch, the rates plain work reaches here beside the published
    peaks.
Inputs are synthetic and seeded.  Usage:
  python bench.py [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-parallel] [--no-backward]
                  [--no-qkv] [--no-long] [--no-small] [--no-peaks] [--copy-mib N]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

MFMA_BF16_PEAK_TFLOPS = 2516.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak


class HipEvents:
    """hipEvent pairs created through the HIP runtime (the library records
    them around its main kernel on the launch stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, i):
        ms = ctypes.c_float(0.0)
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.pairs[i][0]),
                                          ctypes.c_void_p(self.pairs[i][1]))
        if rc:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(ctypes.c_void_p(a))
            self.hip.hipEventDestroy(ctypes.c_void_p(b))


def chunk_flops(T, H, B, dk, dv, b):
    """Algorithmic flops of the whole chunkwise forward."""
    return B * T * H * ((b + 1) * (dk + dv) + 4 * dk * dv)


def chunk_kernel_flops(T, H, B, dk, dv, b):
    """Algorithmic flops of the chunk-recurrence kernel: inter-chunk term and
    state update (2 d_k d_v each) plus the causal value product (b+1) d_v."""
    return B * T * H * (4 * dk * dv + (b + 1) * dv)


def chunk_dense_flops(T, H, B, dk, dv, b):
    """Flops the chunk tiles execute when every intra-chunk product is taken
    over the full b x b block (the causal half included): 2 b (d_k + d_v) +
    4 d_k d_v per token-head."""
    return B * T * H * (2 * b * (dk + dv) + 4 * dk * dv)


def achievable_peaks(torch):
    """Rates this GPU reaches on plain work, as a second scale beside the
    published peaks: a 1 GiB device copy (read + write bytes per second) and
    a large bf16 matrix product through torch (hipBLASLt), 8192^3, both
    operands contiguous.  Median of 10 reps each after 3 warm-ups."""
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    cp = per_call_ms(torch, lambda: dst.copy_(src), 10)
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.mm(a, b, out=c)
    mm = per_call_ms(torch, lambda: torch.mm(a, b, out=c), 10)
    del a, b, c
    copy_gbs = 2 * (1 << 30) / (float(np.median(cp)) / 1e3) / 1e9
    gemm_tflops = 2 * n ** 3 / (float(np.median(mm)) / 1e3) / 1e12
    return {"note": "1 GiB device copy (read + write) and a bf16 8192^3 torch.mm (hipBLASLt); medians of 10 reps",
            "copy_GBs": copy_gbs, "copy_frac_of_peak": copy_gbs / HBM_PEAK_GBS,
            "gemm_tflops": gemm_tflops, "gemm_frac_of_peak": gemm_tflops / MFMA_BF16_PEAK_TFLOPS}


def chunk_bytes(T, H, B, dk, dv):
    """Algorithmic HBM bytes of a bf16 forward: Q, K, V read and O written
    once, plus the fp32 outgoing state."""
    return B * T * H * (2 * dk + 2 * dv) * 2 + B * H * dk * dv * 4


FLUSH_MIB = 512  # larger than the 256 MiB last-level (MALL) cache


class Flusher:
    """Writes a 512 MiB scratch buffer, so that no input of the next call is
    still held in the L2 or last-level cache."""

    def __init__(self, torch):
        self.buf = torch.empty(FLUSH_MIB << 18, dtype=torch.float32, device="cuda:0")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(float(self.i))


def per_call_ms(torch, fn, reps, flush=None):
    """Event-timed duration of each of `reps` calls of fn (a flush, untimed,
    before each when given).  Returns the list of milliseconds."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def stats_ms(ms):
    ms = np.asarray(ms, dtype=np.float64)
    return {"median_ms": float(np.median(ms)), "min_ms": float(ms.min()), "mean_ms": float(ms.mean()),
            "reps": int(ms.size)}


# The sources each measured kernel is built from: its own file, the shared
# device headers and the build script (whose flags shape the generated code).
KERNEL_SOURCES = {
    "chunk_mfma_kernel": "k_chunk_mfma.hip",
    "chunk_ws_kernel": "k_chunk_mfma.hip",
    "chunk_wide_kernel": "k_chunk_wide.hip",
    "chunk_fused_kernel": "k_chunk_fused.hip",
    "prep_kernel": "k_chunk_mfma.hip",
    "gn_finalize_kernel": "k_chunk_mfma.hip",
    "decode_kernel": "k_decode.hip",
}


def kernel_source_sha(kernel):
    """Hash of the sources `kernel` is built from."""
    csrc = ROOT / "retnet_scale_retention_amd" / "csrc"
    h = hashlib.sha256()
    for f in [csrc / KERNEL_SOURCES[kernel]] + sorted(csrc.glob("*.hpp")):
        h.update(f.read_bytes())
    h.update((ROOT / "retnet_scale_retention_amd" / "build.py").read_bytes())
    return h.hexdigest()[:16]


def traffic_record(kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE measurement, if it was taken on the kernel's current sources."""
    p = ROOT / "profiles" / "traffic.json"
    if not p.exists():
        return None
    rec = json.loads(p.read_text()).get(kernel)
    if not rec or rec.get("source_sha") != kernel_source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def call_traffic_record(chunk):
    """HBM bytes of one whole 7B-shaped msr_chunkwise call (every kernel),
    from the committed counter runs, if taken on the current sources."""
    p = ROOT / "profiles" / "traffic.json"
    if not p.exists():
        return None
    rec = json.loads(p.read_text()).get("chunkwise_call_b%d" % chunk)
    if not rec or rec.get("source_sha") != library_source_sha():
        return None
    return rec.get("bytes_per_call")


def library_source_sha():
    """Hash of every library source and the build script."""
    csrc = ROOT / "retnet_scale_retention_amd" / "csrc"
    h = hashlib.sha256()
    for f in sorted(csrc.glob("*.hip")) + sorted(csrc.glob("*.hpp")) + sorted(csrc.glob("*.cpp")):
        h.update(f.read_bytes())
    h.update((ROOT / "retnet_scale_retention_amd" / "build.py").read_bytes())
    return h.hexdigest()[:16]


def bench_chunkwise(torch, msr, mi, steps, warmup, chunk):
    w = mi.WORKLOADS["7b"]
    dev = torch.device("cuda:0")
    q, k, v = mi.qkv(w)
    up = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    qd, kd, vd = up(q), up(k), up(v)
    del q, k, v
    g = mi.gammas(w.H)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g,
                                        msr.MSR_FORM_CHUNKWISE, chunk), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws)
    ev = HipEvents(steps)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # the timed steps: back-to-back calls, with the library recording the
    # main kernel's events (the roofline's kernel time) and nothing else
    t0.record()
    for i in range(steps):
        msr.set_kernel_events(*ev.pairs[i])
        msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws)
    msr.set_kernel_events(None, None)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    kern_ms = [ev.elapsed_ms(i) for i in range(steps)]
    ev.close()
    ms = total_ms / steps
    # per-call durations (median, min) from events around each call, after the timed steps
    call_ms = per_call_ms(torch, lambda: msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws),
                          steps)
    # the same call with a 512 MiB cache flush before each rep
    flushed = stats_ms(per_call_ms(torch, lambda: msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s,
                                                                    workspace=ws), steps, Flusher(torch)))
    # the same call with the split-scores precision option
    wss = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE, chunk,
                                         flags=msr.MSR_FLAG_SPLIT_SCORES), dtype=torch.uint8, device=dev)
    msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=wss, flags=msr.MSR_FLAG_SPLIT_SCORES)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=wss, flags=msr.MSR_FLAG_SPLIT_SCORES)
    t1.record()
    torch.cuda.synchronize()
    split_ms = t0.elapsed_time(t1) / steps
    del wss
    # the other chunk size of the 7B-shaped workload
    ochunk = 256 if chunk != 256 else 128
    wso = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE, ochunk),
                      dtype=torch.uint8, device=dev)
    msr.msr_chunkwise(qd, kd, vd, g, ochunk, out=o, state_out=s, workspace=wso)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        msr.msr_chunkwise(qd, kd, vd, g, ochunk, out=o, state_out=s, workspace=wso)
    t1.record()
    torch.cuda.synchronize()
    other_ms = t0.elapsed_time(t1) / steps
    del wso
    # the fused schedule of the same call
    wsf = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE, chunk,
                                         flags=msr.MSR_FLAG_FUSED), dtype=torch.uint8, device=dev)
    ffn = lambda: msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=wsf, flags=msr.MSR_FLAG_FUSED)
    ffn()
    fused = stats_ms(per_call_ms(torch, ffn, steps))
    del wsf
    kms = float(np.mean(kern_ms))
    flops = chunk_flops(w.T, w.H, w.B, w.dk, w.dv, chunk)
    dflops = chunk_dense_flops(w.T, w.H, w.B, w.dk, w.dv, chunk)
    kflops = chunk_kernel_flops(w.T, w.H, w.B, w.dk, w.dv, chunk)
    return {
        "workload": w, "chunk": chunk, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms / 1e3),
        "kernel_ms": kms, "flops": flops, "dense_flops": dflops, "kernel_flops": kflops, "split_scores_ms": split_ms,
        "other_chunk": {"chunk": ochunk, "ms_per_step": other_ms, "tokens_per_s": w.B * w.T / (other_ms / 1e3),
                        "step_tflops": chunk_flops(w.T, w.H, w.B, w.dk, w.dv, ochunk) / (other_ms / 1e3) / 1e12},
        "bytes": chunk_bytes(w.T, w.H, w.B, w.dk, w.dv),
        "kernel_tflops": kflops / (kms / 1e3) / 1e12, "step_tflops": flops / (ms / 1e3) / 1e12,
        "call": stats_ms(call_ms), "kernel": stats_ms(kern_ms), "flushed": flushed,
        "fused": {**fused, "tokens_per_s": w.B * w.T / (fused["median_ms"] / 1e3)},
    }


def bench_long(torch, msr, mi, calls):
    """The long-sequence workload's chunk sweep: one state carried across all
    chunks of each (batch, head) pair."""
    w = mi.WORKLOADS["long"]
    dev = torch.device("cuda:0")
    q, k, v = mi.qkv(w)
    up = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    qd, kd, vd = up(q), up(k), up(v)
    del q, k, v
    g = mi.gammas(w.H)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    out = {"config": {"B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv}}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    nbytes = chunk_bytes(w.T, w.H, w.B, w.dk, w.dv)
    out["bytes_per_call"] = nbytes
    for chunk in w.chunks:
        ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE,
                                            chunk), dtype=torch.uint8, device=dev)
        fn = lambda: msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws)
        fn()
        st = stats_ms(per_call_ms(torch, fn, calls))
        ms = st["median_ms"]
        del ws
        out["b%d" % chunk] = {"ms_per_call": ms, **st, "tokens_per_s": w.B * w.T / (ms / 1e3),
                              "step_tflops": chunk_flops(w.T, w.H, w.B, w.dk, w.dv, chunk) / (ms / 1e3) / 1e12,
                              "hbm_GBs": nbytes / (ms / 1e3) / 1e9,
                              "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
        if chunk in (64, 128):  # the fused schedule at the same chunk
            fl = msr.MSR_FLAG_FUSED
            ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE,
                                                chunk, flags=fl), dtype=torch.uint8, device=dev)
            fn = lambda: msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws, flags=fl)
            fn()
            st = stats_ms(per_call_ms(torch, fn, calls))
            ms = st["median_ms"]
            del ws
            out["b%d" % chunk]["fused"] = {"ms_per_call": ms, **st, "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
    return out


def bench_small(torch, msr, mi, reps):
    """The small model layer (B=4, T=2048, H=8, d_k=d_v=64, chunk 64, bf16):
    its 34 MB of inputs and outputs fit the last-level cache, so a 512 MiB
    flush precedes every timed call."""
    w = mi.WORKLOADS["small"]
    dev = torch.device("cuda:0")
    q, k, v = mi.qkv(w)
    up = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    qd, kd, vd = up(q), up(k), up(v)
    g = mi.gammas(w.H)
    chunk = w.chunks[0]
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE,
                                               chunk)), dtype=torch.uint8, device=dev)
    fn = lambda: msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws)
    for _ in range(3):
        fn()
    fl = stats_ms(per_call_ms(torch, fn, reps, Flusher(torch)))
    warm = stats_ms(per_call_ms(torch, fn, reps))
    nbytes = chunk_bytes(w.T, w.H, w.B, w.dk, w.dv)
    ms = fl["median_ms"]
    return {"config": {"workload": "small model layer", "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                       "chunk": chunk, "dtype": "bf16"},
            "flushed": fl, "warm": warm, "tokens_per_s": w.B * w.T / (ms / 1e3),
            "bytes_per_call": nbytes, "hbm_GBs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "step_tflops": chunk_flops(w.T, w.H, w.B, w.dk, w.dv, chunk) / (ms / 1e3) / 1e12}


def bench_parallel(torch, msr, mi, steps):
    """The parallel form over the 7B-shaped layer (same inputs as the chunkwise leg)."""
    w = mi.WORKLOADS["7b"]
    dev = torch.device("cuda:0")
    q, k, v = mi.qkv(w)
    up = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    qd, kd, vd = up(q), up(k), up(v)
    del q, k, v
    g = mi.gammas(w.H)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g,
                                        msr.MSR_FORM_PARALLEL, 0), dtype=torch.uint8, device=dev)
    msr.msr_parallel(qd, kd, vd, g, out=o, state_out=s, workspace=ws)
    ev = HipEvents(steps)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        msr.set_kernel_events(*ev.pairs[i])
        msr.msr_parallel(qd, kd, vd, g, out=o, state_out=s, workspace=ws)
    msr.set_kernel_events(None, None)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kms = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    th = w.B * w.T * w.H
    flops = th * ((w.T + 1) * (w.dk + w.dv) + 4 * w.dk * w.dv)
    kflops = th * ((w.T + 1) * (w.dk + w.dv) + 2 * w.dk * w.dv)  # output kernel: scores, values, S_in term
    return {"config": {"B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv}, "ms_per_call": ms,
            "tokens_per_s": w.B * w.T / (ms / 1e3), "tflops": flops / (ms / 1e3) / 1e12,
            "kernel": "parallel_mfma_kernel", "kernel_us": kms * 1e3,
            "kernel_tflops": kflops / (kms / 1e3) / 1e12,
            "kernel_mfma_frac": kflops / (kms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def bench_backward(torch, msr, mi, name, calls, chunk):
    """The backward pass (msr_chunkwise_backward) on a workload: gradients of
    L = sum(O dO) + sum(S_out dS_out) with respect to Q, K, V and S_in."""
    w = mi.WORKLOADS[name]
    dev = torch.device("cuda:0")
    g = mi.gammas(w.H)
    shp = lambda d: (w.B, w.T, w.H, d)
    q = mi.device_normal(shp(w.dk), 4001, dev, torch.bfloat16)
    k = mi.device_normal(shp(w.dk), 4002, dev, torch.bfloat16)
    v = mi.device_normal(shp(w.dv), 4003, dev, torch.bfloat16)
    do = mi.device_normal(shp(w.dv), 4004, dev, torch.bfloat16)
    ds = mi.device_normal((w.B, w.H, w.dk, w.dv), 4005, dev, torch.float32)
    ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_BACKWARD,
                                        chunk), dtype=torch.uint8, device=dev)
    msr.msr_chunkwise_backward(q, k, v, g, chunk, do, grad_state=ds, workspace=ws)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(calls):
        msr.msr_chunkwise_backward(q, k, v, g, chunk, do, grad_state=ds, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / calls
    th = w.B * w.T * w.H
    # algorithmic flops: three retention products, each (b+1)(d1+d2) + 4 d1 d2 per token-head
    flops = th * (2 * ((chunk + 1) * (w.dv + w.dk) + 4 * w.dv * w.dk) + (chunk + 1) * (w.dk + w.dv) + 4 * w.dk * w.dv)
    return {"config": {"workload": name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv, "chunk": chunk,
                       "dtype": "bf16", "workspace_bytes": int(ws.numel())},
            "ms_per_call": ms, "tokens_per_s": w.B * w.T / (ms / 1e3), "tflops": flops / (ms / 1e3) / 1e12}


def bench_qkv(torch, msr, mi, calls, chunk):
    """The Q/K/V projections (bf16 MFMA GEMM with the rotation in its
    epilogue) over the 7B-shaped layer input, d_model = H d_k = 4096, and the
    composite projections + chunkwise form."""
    w = mi.WORKLOADS["7b"]
    dev = torch.device("cuda:0")
    dm = w.H * w.dk
    g = mi.gammas(w.H)
    x = mi.device_normal((w.B, w.T, dm), 7001, dev, torch.bfloat16)
    wts = [(mi.device_normal((w.H * d, dm), 7002 + i, dev, torch.float32) / np.sqrt(dm)).to(torch.bfloat16)
           for i, d in enumerate((w.dk, w.dk, w.dv))]
    out = (torch.empty((w.B, w.T, w.H, w.dk), dtype=torch.bfloat16, device=dev),
           torch.empty((w.B, w.T, w.H, w.dk), dtype=torch.bfloat16, device=dev),
           torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev))
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_QKV_CHUNKWISE,
                                        chunk), dtype=torch.uint8, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(calls):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / calls

    ms_p = timed(lambda: msr.msr_qkv_projection(x, *wts, w.H, out=out))
    ms_l = timed(lambda: msr.msr_qkv_chunkwise(x, *wts, g, chunk, out=o, state_out=s, workspace=ws))
    flops = 2.0 * w.B * w.T * dm * w.H * (2 * w.dk + w.dv)
    return {"config": {"workload": "7B-shaped layer input", "B": w.B, "T": w.T, "d_model": dm, "H": w.H,
                       "dk": w.dk, "dv": w.dv, "chunk": chunk, "dtype": "bf16"},
            "projection_ms": ms_p, "projection_tflops": flops / (ms_p / 1e3) / 1e12,
            "projection_mfma_frac": flops / (ms_p / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "layer_ms": ms_l, "layer_tokens_per_s": w.B * w.T / (ms_l / 1e3)}


def bench_decode(torch, msr, mi, nsteps):
    w = mi.WORKLOADS["decode"]
    dev = torch.device("cuda:0")
    g = mi.gammas(w.H)
    # prefill (chunkwise, chunk 128) seeds the state
    q = mi.device_normal((w.B, w.T, w.H, w.dk), 3001, dev, torch.bfloat16)
    k = mi.device_normal((w.B, w.T, w.H, w.dk), 3002, dev, torch.bfloat16)
    v = mi.device_normal((w.B, w.T, w.H, w.dv), 3003, dev, torch.bfloat16)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    _, state = msr.msr_chunkwise(q, k, v, g, 128)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - tp0) * 1e3
    del q, k, v
    qs = mi.device_normal((nsteps, w.B, w.H, w.dk), 3004, dev, torch.bfloat16)
    ks = mi.device_normal((nsteps, w.B, w.H, w.dk), 3005, dev, torch.bfloat16)
    vs = mi.device_normal((nsteps, w.B, w.H, w.dv), 3006, dev, torch.bfloat16)
    o = torch.empty((w.B, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    for i in range(3):  # warm-up on a copy of the state
        st = state.clone()
        msr.msr_recurrent_step(qs[i], ks[i], vs[i], st, g, w.T + i, out=o)
    ev = HipEvents(nsteps)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(nsteps):
        msr.set_kernel_events(*ev.pairs[i])
        msr.msr_recurrent_step(qs[i], ks[i], vs[i], state, g, w.T + i, out=o)
    msr.set_kernel_events(None, None)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    kern = [ev.elapsed_ms(i) for i in range(nsteps)]
    ev.close()
    step_ms = total_ms / nsteps
    kms = float(np.mean(kern))
    bytes_step = 2 * w.B * w.H * w.dk * w.dv * 4 + w.B * w.H * (2 * w.dk + 2 * w.dv) * 2

    # the same step loop captured once in a HIP graph (each step's position is
    # a kernel argument of its own node), replayed: no host launch gaps
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        for i in range(nsteps):
            msr.msr_recurrent_step(qs[i], ks[i], vs[i], state, g, w.T + i, out=o)
    gph.replay()
    torch.cuda.synchronize()
    graph_ms = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gph.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms.append(a.elapsed_time(b) / nsteps)
    del gph
    gstep = float(np.median(graph_ms))

    # batched serving: every sequence at its own position (one per batch row)
    nr = max(8, nsteps // 8)
    base = torch.tensor([(b * 37) % 4096 for b in range(w.B)], dtype=torch.int64, device=dev)
    pos = [base + w.T + i for i in range(nr)]
    evr = HipEvents(nr)
    torch.cuda.synchronize()
    for i in range(nr):
        msr.set_kernel_events(*evr.pairs[i])
        msr.msr_recurrent_step(qs[i], ks[i], vs[i], state, g, pos[i], out=o)
    msr.set_kernel_events(None, None)
    torch.cuda.synchronize()
    rk = float(np.mean([evr.elapsed_ms(i) for i in range(nr)]))
    evr.close()
    # multi-token steps: 4 new tokens per sequence per call (chunkwise, chunk 4, state carried)
    tq = mi.device_normal((w.B, 4, w.H, w.dk), 3007, dev, torch.bfloat16)
    tk = mi.device_normal((w.B, 4, w.H, w.dk), 3008, dev, torch.bfloat16)
    tv = mi.device_normal((w.B, 4, w.H, w.dv), 3009, dev, torch.bfloat16)
    ws = torch.empty(msr.workspace_size(w.B, 4, w.H, w.dk, w.dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE, 4),
                     dtype=torch.uint8, device=dev)
    mo = torch.empty((w.B, 4, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    msr.msr_chunkwise(tq, tk, tv, g, 4, state_in=state, state_out=state, out=mo, workspace=ws, pos_rows=pos[0])
    nm = 8
    torch.cuda.synchronize()
    tm0 = time.perf_counter()
    for i in range(nm):
        msr.msr_chunkwise(tq, tk, tv, g, 4, state_in=state, state_out=state, out=mo, workspace=ws,
                          pos_rows=pos[0] + 4 * i)
    torch.cuda.synchronize()
    mms = (time.perf_counter() - tm0) * 1e3 / nm
    return {
        "config": {"B": w.B, "H": w.H, "dk": w.dk, "dv": w.dv, "prefill_tokens": w.T, "steps": nsteps},
        "note": "steps_per_s: wall time of the step loop captured in a HIP graph and replayed (median of 3 "
                "replays); eager: the same loop launched from the host",
        "steps_per_s": 1e3 / gstep, "tokens_per_s": w.B * 1e3 / gstep, "ms_per_step": gstep,
        "wall_hbm_frac": bytes_step / (gstep / 1e3) / 1e9 / HBM_PEAK_GBS,
        "eager": {"steps_per_s": 1e3 / step_ms, "ms_per_step": step_ms},
        "kernel_us": kms * 1e3,
        "hbm": {"achieved": bytes_step / (kms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": bytes_step / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, "bytes_per_step": bytes_step,
                "traffic": traffic_record("decode_kernel")},
        "prefill_ms": prefill_ms,
        "ragged": {"note": "one position per batch row", "steps": nr, "kernel_us": rk * 1e3,
                   "steps_per_s": 1e3 / rk, "hbm_frac": bytes_step / (rk / 1e3) / 1e9 / HBM_PEAK_GBS},
        "multi_token": {"note": "4 tokens per sequence per call (msr_chunkwise, b=4: one pass over the state "
                                "for all 4 tokens), rows at their own positions", "calls": nm, "ms_per_call": mms,
                        "tokens_per_s": w.B * 4 * 1e3 / mms},
    }


def cpu_baseline(mi, chunk):
    """The oracle's chunkwise form on a bounded sample of the 7B workload:
    16 (batch, head) pairs x 8192 tokens, scaled linearly to the full B*T*H
    token-heads (the form's cost is linear in tokens and pairs)."""
    from oracle import oracle
    w = mi.WORKLOADS["7b"]
    Ts, Hs = 8192, 16
    q, k, v = mi.qkv(w, T=Ts)
    q, k, v = (x[:1, :, :Hs] for x in (q, k, v))
    g = mi.gammas(w.H)[:Hs]
    t0 = time.perf_counter()
    oracle.chunkwise(q, k, v, g, chunk)
    dt = time.perf_counter() - t0
    token_heads = Ts * Hs
    full = w.B * w.T * w.H
    tokens_per_s = w.B * w.T / (dt * full / token_heads)
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"chunkwise form, chunk {chunk}, {Hs} heads x {Ts} tokens of the 7B-shaped layer "
                      f"({dt:.1f} s), scaled to B*T*H = {full} token-heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the warm-up is long enough (about 40 ms of calls) for the GPU to reach its
    # steady clocks: the first tens of calls after a pause run up to 10% slower
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--chunk", type=int, default=128)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-qkv", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-parallel", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run 3 plain device copies of this many MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the operator runs on a single MI355X here "
              "(the (batch, head) pairs would shard across GPUs with no communication); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import msr_inputs as mi
    import retnet_scale_retention_amd as msr
    msr.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    r = bench_chunkwise(torch, msr, mi, args.steps, args.warmup, args.chunk)
    w = r["workload"]
    lng = None if args.no_long else bench_long(torch, msr, mi, 7)
    sml = None if args.no_small else bench_small(torch, msr, mi, 20)
    dec = None if args.no_decode else bench_decode(torch, msr, mi, args.decode_steps)
    par = None if args.no_parallel else bench_parallel(torch, msr, mi, 3)
    bwd = None
    if not args.no_backward:
        bwd = {"small": bench_backward(torch, msr, mi, "small", 3, 64),
               "7b": bench_backward(torch, msr, mi, "7b", 5, 128)}
    qkv = None if args.no_qkv else bench_qkv(torch, msr, mi, 5, args.chunk)
    peaks = None if args.no_peaks else achievable_peaks(torch)
    cpu = None if args.no_cpu else cpu_baseline(mi, args.chunk)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the 7B-shaped layer's chunk recurrence runs as the warp-specialised
    # kernel at b = 64 and 128 and as the single-role kernel at b = 256
    main_kernel = "chunk_ws_kernel" if args.chunk <= 128 else "chunk_mfma_kernel"
    traffic = traffic_record(main_kernel)
    line = {
        "metric": "chunkwise MSR fwd tokens/s + decode steps/s; % of bf16 MFMA / HBM peak",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7B-shaped MSR layer chunkwise forward", "B": w.B, "T": w.T, "H": w.H,
                   "dk": w.dk, "dv": w.dv, "chunk": r["chunk"], "state": "fp32"},
        "roofline": {"bound": "mfma", "achieved": r["kernel_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": r["kernel_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic, "kernel": main_kernel,
                     "kernel_us": r["kernel_ms"] * 1e3, "flops_per_launch": r["kernel_flops"]},
        "step_tflops": r["step_tflops"], "step_mfma_frac": r["step_tflops"] / MFMA_BF16_PEAK_TFLOPS,
        "call_roofline": {
            "note": "the whole call (every kernel of one msr_chunkwise), algorithmic flops "
                    "(b+1)(dk+dv) + 4 dk dv per token-head over the event-timed call; traffic: the call's "
                    "counter bytes (all kernels) against its algorithmic bytes",
            "achieved": r["flops"] / (r["call"]["median_ms"] / 1e3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": r["flops"] / (r["call"]["median_ms"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "flops_per_call": r["flops"], "algorithmic_bytes": r["bytes"],
            "traffic": call_traffic_record(r["chunk"]),
            "dense_chunk": {"note": "flops the full b x b intra-chunk tiles execute, 2b(dk+dv) + 4 dk dv per "
                                    "token-head, over the same call time",
                            "flops_per_call": r["dense_flops"],
                            "tflops": r["dense_flops"] / (r["call"]["median_ms"] / 1e3) / 1e12}},
        "achievable_peaks": peaks,
        "timing": {"call": r["call"], "kernel": r["kernel"], "flushed_call": r["flushed"]},
        "small_layer": sml,
        "split_scores": {"note": "the same call with MSR_FLAG_SPLIT_SCORES (precision option for strong decay)",
                         "ms_per_step": r["split_scores_ms"]},
        "other_chunk": r["other_chunk"],
        "fused_schedule": {"note": "the same call with MSR_FLAG_FUSED (opt-in schedule)", **r["fused"]},
        "long_sequence": lng,
        "cpu_baseline": cpu,
        "decode": dec,
        "parallel": par,
        "backward": bwd,
        "qkv": qkv,
        "hbm_view": {"bytes_per_step": r["bytes"],
                     "achieved_GBs": r["bytes"] / (r["ms_per_step"] / 1e3) / 1e9,
                     "frac": r["bytes"] / (r["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
