"""Gradients of multi-scale retention for the fp64 oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It writes the plain parallel
definition -- rotation, scale, decay mask, the incoming-state term, the
outgoing state, the optional row-normalised decay and GroupNorm -- with
torch CPU float64 operations and lets
torch.autograd differentiate it.  It shares nothing with the HIP library.
Its forward values are pinned against the C oracle (oracle.c, an independent
implementation) and its gradients against central finite differences of the
C oracle's forward, in tests/test_oracle_pins.py.

Page references (by site and section):
  jsqmd.com "From RoPE to Retention" -- s2 theta_shift rotation, s3 decay
      mask, s4.1 parallel form with the incoming state, s5 GroupNorm, the
      1/sqrt(d) scale and the per-row normalisation of the decay weights.
  aiqz.cc RetNet tutorial -- decay mask and parallel representation.
Parameters held as fp32 on the GPU side (gamma, theta, scale, eps) are the
same fp32 values here, promoted.
"""
from __future__ import annotations

import numpy as np

from oracle.oracle import default_scale, default_theta


def _torch():
    import torch
    return torch


def _rotate(x, theta, pos):
    """theta_shift of x [B, T, H, dk] with row b's token t at position
    pos[b] + t: pair i -> (x0 c - x1 s, x1 c + x0 s), angle = position theta_i."""
    torch = _torch()
    B, T, H, dk = x.shape
    p = pos[:, None] + torch.arange(T, dtype=torch.float64)[None, :]          # [B, T]
    phi = p[:, :, None, None] * theta[None, None, None, :]                    # [B, T, 1, dk/2]
    c, s = torch.cos(phi), torch.sin(phi)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = torch.stack((x0 * c - x1 * s, x1 * c + x0 * s), dim=-1)             # [..., dk/2, 2]
    return y.reshape(B, T, H, dk)


def _forward(q, k, v, s_in, gamma, theta, scale, eps, pos, rotate, groupnorm, rownorm=False):
    torch = _torch()
    B, T, H, dk = q.shape
    qr = _rotate(q, theta, pos) if rotate else q
    kr = (_rotate(k, theta, pos) if rotate else k) * scale
    n = torch.arange(T, dtype=torch.float64)
    diff = n[:, None] - n[None, :]                                            # n - m
    g = gamma[:, None, None]                                                  # [H, 1, 1]
    D = torch.where(diff[None] >= 0, g ** diff.clamp(min=0)[None], torch.zeros((), dtype=torch.float64))
    A = torch.einsum("bnhd,bmhd->bhnm", qr, kr) * D[None]                     # [B, H, T, T]
    o = torch.einsum("bhnm,bmhe->bnhe", A, v)
    s_out = torch.einsum("bmhd,bmhe,hm->bhde", kr, v, gamma[:, None] ** (T - 1 - n)[None, :])
    if s_in is not None:
        xi = gamma[None, :] ** (n[:, None] + 1)                               # [T, H]: gamma^(n+1)
        o = o + xi[None, :, :, None] * torch.einsum("bnhd,bhde->bnhe", qr, s_in)
        s_out = s_out + (gamma ** T)[None, :, None, None] * s_in
    if rownorm:
        # each decay row divided by its sum over absolute positions 0 .. p:
        # sum_j gamma^j for j = 0 .. p, added term by term as in the C oracle
        p = pos[:, None] + n[None, :]                                          # [B, T]
        r = torch.stack([torch.stack([
            (gamma[h] ** torch.arange(int(p[b, t]) + 1, dtype=torch.float64)).sum()
            for h in range(H)]) for b in range(B) for t in range(T)]).reshape(B, T, H)
        o = o / r[..., None]
    if groupnorm:
        mean = o.mean(dim=-1, keepdim=True)
        var = ((o - mean) ** 2).mean(dim=-1, keepdim=True)
        o = (o - mean) / torch.sqrt(var + eps)
    return o, s_out


def _args(q, gamma, theta, scale, eps, pos0, pos_rows):
    torch = _torch()
    dk = q.shape[3]
    th = default_theta(dk) if theta is None else np.asarray(theta, np.float32)
    sc = default_scale(dk) if scale is None else float(np.float32(scale))
    pos = (np.full(q.shape[0], pos0, np.int64) if pos_rows is None else np.asarray(pos_rows, np.int64))
    return (torch.tensor(np.asarray(gamma, np.float32).astype(np.float64)),
            torch.tensor(th.astype(np.float64)), sc, float(np.float32(eps)),
            torch.tensor(pos.astype(np.float64)))


def _t(x, grad=False):
    torch = _torch()
    if x is None:
        return None
    return torch.tensor(np.asarray(x, np.float64), requires_grad=grad)


def forward(q, k, v, gamma, *, s_in=None, theta=None, scale=None, eps=1e-5, pos0=0, pos_rows=None,
            rotate=True, groupnorm=True, rownorm=False):
    """The parallel definition.  q, k: [B, T, H, dk]; v: [B, T, H, dv];
    pos_rows: optional per-batch-row start positions.  Returns (O, S_out)."""
    g, th, sc, ep, pos = _args(q, gamma, theta, scale, eps, pos0, pos_rows)
    o, s = _forward(_t(q), _t(k), _t(v), _t(s_in), g, th, sc, ep, pos, rotate, groupnorm, rownorm)
    return o.detach().numpy(), s.detach().numpy()


def backward(q, k, v, gamma, grad_out, *, grad_state=None, s_in=None, theta=None, scale=None, eps=1e-5,
             pos0=0, pos_rows=None, rotate=True, groupnorm=True, rownorm=False):
    """Gradients of L = sum(O * grad_out) + sum(S_out * grad_state) with
    respect to q, k, v and s_in (a zero incoming state when s_in is None).
    Returns (dq, dk, dv, ds_in) as float64 arrays."""
    torch = _torch()
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[3]
    g, th, sc, ep, pos = _args(q, gamma, theta, scale, eps, pos0, pos_rows)
    tq, tk, tv = _t(q, True), _t(k, True), _t(v, True)
    ts = _t(np.zeros((B, H, dk, dv)) if s_in is None else s_in, True)
    o, s = _forward(tq, tk, tv, ts, g, th, sc, ep, pos, rotate, groupnorm, rownorm)
    loss = (o * _t(grad_out)).sum()
    if grad_state is not None:
        loss = loss + (s * _t(grad_state)).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (tq, tk, tv, ts))
