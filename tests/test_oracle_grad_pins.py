"""Pins of the oracle's gradients (oracle/grad.py: the parallel definition in
torch float64, differentiated by autograd).

- Its forward values equal the C oracle's (oracle.c), an independent
  implementation, for every option the backward pass takes.
- Its gradients equal central finite differences of the C oracle's forward
  along random directions, for Q, K, V and the incoming state, with and
  without GroupNorm and rotation, and with the row-normalised decay.
- With one token, no rotation and no GroupNorm the gradients have a closed
  form, checked directly.
"""
import numpy as np
import pytest

from oracle import grad as og
from oracle import oracle as orc


def rel(x, r):
    return float(np.max(np.abs(np.asarray(x) - np.asarray(r))) / max(np.max(np.abs(r)), 1e-300))


def inputs(seed, B=2, T=12, H=2, dk=8, dv=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk)),
            rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, H, dk, dv)))


GAMMA = np.array([0.96875, 0.75], np.float32)


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("groupnorm", [True, False])
@pytest.mark.parametrize("with_state", [True, False])
@pytest.mark.parametrize("rownorm", [False, True])
def test_forward_matches_the_c_oracle(rotate, groupnorm, with_state, rownorm):
    q, k, v, s = inputs(1)
    s = s if with_state else None
    kw = dict(s_in=s, pos0=7, rotate=rotate, groupnorm=groupnorm, rownorm=rownorm)
    ro, rs = orc.parallel(q, k, v, GAMMA, **kw)
    o, so = og.forward(q, k, v, GAMMA, **kw)
    assert rel(o, ro) < 1e-12 and rel(so, rs) < 1e-12


def test_forward_row_positions_match_the_c_oracle_per_row():
    q, k, v, s = inputs(2, B=3)
    pos = [0, 100, 9]
    o, so = og.forward(q, k, v, GAMMA, s_in=s, pos_rows=pos)
    for b in range(3):
        ro, rs = orc.parallel(q[b:b + 1], k[b:b + 1], v[b:b + 1], GAMMA, s_in=s[b:b + 1], pos0=pos[b])
        assert rel(o[b:b + 1], ro) < 1e-12 and rel(so[b:b + 1], rs) < 1e-12


def loss_c(q, k, v, s, do, ds, **kw):
    """L = sum(O dO) + sum(S_out dS) with the C oracle's forward."""
    o, so = orc.parallel(q, k, v, GAMMA, s_in=s, **kw)
    return float(np.sum(o * do) + np.sum(so * ds))


@pytest.mark.parametrize("rotate,groupnorm,rownorm", [(True, True, False), (False, True, False),
                                                      (True, False, False), (True, True, True),
                                                      (True, False, True)])
def test_gradients_match_finite_differences_of_the_c_oracle(rotate, groupnorm, rownorm):
    q, k, v, s = inputs(3)
    rng = np.random.default_rng(30)
    do = rng.standard_normal(q.shape[:3] + (v.shape[3],))
    ds = rng.standard_normal(s.shape)
    kw = dict(pos0=5, rotate=rotate, groupnorm=groupnorm, rownorm=rownorm)
    grads = og.backward(q, k, v, GAMMA, do, grad_state=ds, s_in=s, **kw)
    base = [q, k, v, s]
    for i, gr in enumerate(grads):
        for trial in range(3):
            e = rng.standard_normal(base[i].shape)
            eps = 1e-5
            xp = [x.copy() for x in base]
            xm = [x.copy() for x in base]
            xp[i] = xp[i] + eps * e
            xm[i] = xm[i] - eps * e
            fd = (loss_c(*xp, do, ds, **kw) - loss_c(*xm, do, ds, **kw)) / (2 * eps)
            an = float(np.sum(gr * e))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, trial, fd, an)


def test_single_token_closed_form():
    # T = 1, no rotation, no GroupNorm:
    #   O = s (q.k) v + g q S,  S_out = g S + s k^T v
    rng = np.random.default_rng(4)
    dk, dv = 6, 5
    q, k = rng.standard_normal((1, 1, 1, dk)), rng.standard_normal((1, 1, 1, dk))
    v = rng.standard_normal((1, 1, 1, dv))
    S = rng.standard_normal((1, 1, dk, dv))
    do = rng.standard_normal((1, 1, 1, dv))
    dS = rng.standard_normal((1, 1, dk, dv))
    g = np.float32(0.875)
    sc = float(np.float32(1 / np.sqrt(dk)))
    dq, dk_, dvv, dsi = og.backward(q, k, v, [g], do, grad_state=dS, s_in=S, rotate=False, groupnorm=False)
    qv, kv, vv, dov, Sv, dSv = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], do[0, 0, 0], S[0, 0], dS[0, 0]
    gg = float(g)
    assert np.allclose(dq[0, 0, 0], sc * (dov @ vv) * kv + gg * Sv @ dov, rtol=1e-13, atol=1e-13)
    assert np.allclose(dk_[0, 0, 0], sc * (dov @ vv) * qv + sc * dSv @ vv, rtol=1e-13, atol=1e-13)
    assert np.allclose(dvv[0, 0, 0], sc * (qv @ kv) * dov + sc * dSv.T @ kv, rtol=1e-13, atol=1e-13)
    assert np.allclose(dsi[0, 0], gg * np.outer(qv, dov) + gg * dSv, rtol=1e-13, atol=1e-13)
