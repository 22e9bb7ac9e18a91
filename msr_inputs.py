"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no retention arithmetic.  It draws N(0, 1) samples from
numpy's PCG64 generator keyed by (workload, tensor id, ...), rounds them to
bf16 (round-to-nearest-even) where the workload is bf16, and lists the
workload shapes.  The per-head decay values gamma_h = 1 - 2^(-5-h) are part
of each workload's description and are provided here as data.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# tensor ids used as the second seed word
Q, K, V, S_IN = 0, 1, 2, 3
DECODE_BASE = 100  # decode step s draws q, k, v with ids 100 + 3 s + {0, 1, 2}


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str  # "f32" or "bf16"
    chunks: tuple


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 64, 2, 16, 16, "f32", (1, 16, 64)),
    "small": Workload("small", 1, 4, 2048, 8, 64, 64, "bf16", (64,)),
    "7b": Workload("7b", 2, 2, 8192, 16, 256, 512, "bf16", (128, 256)),
    # decode: prefill of T tokens (chunk 128), then single-token steps
    "decode": Workload("decode", 3, 64, 2048, 16, 256, 512, "bf16", (128,)),
    "long": Workload("long", 4, 1, 131072, 8, 128, 256, "bf16", (64, 128, 256)),
}

DECODE_STEPS = 1024


def gammas(H: int) -> np.ndarray:
    """Per-head decay of the workloads: gamma_h = 1 - 2^(-5-h) (fp32, exact)."""
    return (1.0 - np.exp2(-5.0 - np.arange(H, dtype=np.float64))).astype(np.float32)


def normal(key, shape) -> np.ndarray:
    """float32 N(0, 1) samples from PCG64 seeded with the integer list `key`."""
    return np.random.default_rng(list(key)).standard_normal(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Values of x rounded to bf16, held exactly in float32."""
    return bf16_to_f32(bf16_bits(x))


def quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def tensor(w: Workload, tid: int, d: int, T: int | None = None, per_slice: bool = False):
    """One [B, T, H, d] input tensor of workload w (values already in w.dtype).

    per_slice=True draws each (b, h) slice from its own key so that a single
    slice can be regenerated alone (used for the very large decode prefill)."""
    T = w.T if T is None else T
    if not per_slice:
        return quantize(normal((w.seed, tid), (w.B, T, w.H, d)), w.dtype)
    out = np.empty((w.B, T, w.H, d), dtype=np.float32)
    for b in range(w.B):
        for h in range(w.H):
            out[b, :, h, :] = slice_tensor(w, tid, d, b, h, T)
    return out


def slice_tensor(w: Workload, tid: int, d: int, b: int, h: int, T: int | None = None):
    """The (b, h) slice [T, d] of a per_slice tensor."""
    T = w.T if T is None else T
    return quantize(normal((w.seed, tid, b, h), (T, d)), w.dtype)


def qkv(w: Workload, T: int | None = None, per_slice: bool = False):
    return (tensor(w, Q, w.dk, T, per_slice), tensor(w, K, w.dk, T, per_slice),
            tensor(w, V, w.dv, T, per_slice))


def decode_token(w: Workload, s: int):
    """q, k: [B, H, dk]; v: [B, H, dv] for decode step s."""
    base = DECODE_BASE + 3 * s
    return (quantize(normal((w.seed, base), (w.B, w.H, w.dk)), w.dtype),
            quantize(normal((w.seed, base + 1), (w.B, w.H, w.dk)), w.dtype),
            quantize(normal((w.seed, base + 2), (w.B, w.H, w.dv)), w.dtype))


def state(w: Workload, scale: float = 1.0):
    """A seeded fp32 incoming state [B, H, dk, dv]."""
    return (normal((w.seed, S_IN), (w.B, w.H, w.dk, w.dv)) * np.float32(scale)).astype(np.float32)


def device_normal(shape, seed: int, device, dtype):
    """N(0, 1) tensor drawn on the device by torch's Philox generator seeded
    with `seed` (for inputs too large to draw on the host), cast to dtype."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)
