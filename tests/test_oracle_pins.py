"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these re-types the oracle's loops: each checks a closed form, an
invariant the pages state, a library routine, or an independent formulation
(complex-number rotation, dense decay-mask matrix) on tiny inputs.
"""
import json
from pathlib import Path

import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc

GOLDEN = Path(__file__).resolve().parent / "golden"


def rel(x, r):
    return float(np.max(np.abs(np.asarray(x) - np.asarray(r))) / max(np.max(np.abs(r)), 1e-300))


def tiny(seed=7, B=1, T=64, H=2, dk=16, dv=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    s = rng.standard_normal((B, H, dk, dv))
    return q, k, v, s


# ---------------------------------------------------------------- page demo
def test_demo_parallel_equals_recurrent_within_page_bound():
    """aiqz.cc 'Python demo': parallel and recurrent retention agree to < 1e-8
    at n=8, dim=6, gamma=0.9 (no rotation, no scale, no GroupNorm)."""
    g = json.loads((GOLDEN / "demo_parallel_vs_recurrent.json").read_text())
    n, d = g["n"], g["dim"]
    rng = np.random.default_rng(42)
    x = rng.standard_normal((n, d))
    wq, wk, wv = (rng.standard_normal((d, d)) for _ in range(3))
    q, k, v = (x @ w for w in (wq, wk, wv))
    shp = lambda a: a[None, :, None, :]
    kw = dict(rotate=False, scale=g["scale"], groupnorm=False)
    op, sp = orc.parallel(shp(q), shp(k), shp(v), [g["gamma"]], **kw)
    orr, sr = orc.recurrent(shp(q), shp(k), shp(v), [g["gamma"]], **kw)
    assert np.max(np.abs(op - orr)) < g["max_abs_err_bound"]
    assert np.max(np.abs(sp - sr)) < g["max_abs_err_bound"]


# ------------------------------------------------------- three-form identity
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("groupnorm", [False, True])
def test_three_forms_agree_for_every_chunk(with_state, groupnorm):
    """The parallel, recurrent and chunkwise forms are the same function
    (jsqmd.com s4; aiqz.cc 'recurrent representation'; b99b.cn)."""
    q, k, v, s = tiny()
    g = mi.gammas(2)
    s_in = s if with_state else None
    kw = dict(s_in=s_in, groupnorm=groupnorm, pos0=5)
    op, sp = orc.parallel(q, k, v, g, **kw)
    orr, sr = orc.recurrent(q, k, v, g, **kw)
    assert rel(orr, op) < 1e-12 and rel(sr, sp) < 1e-12
    for c in (1, 2, 4, 8, 16, 32, 64):
        oc, sc = orc.chunkwise(q, k, v, g, c, **kw)
        assert rel(oc, op) < 1e-12, c
        assert rel(sc, sp) < 1e-12, c


def test_chunk_1_is_recurrence_and_chunk_T_is_parallel():
    """b=1 reduces to the recurrence, b=n to the parallel form (aiqz.cc
    'chunkwise recurrence')."""
    q, k, v, s = tiny(seed=3, T=24)
    g = [0.9, 0.5]
    o1, s1 = orc.chunkwise(q, k, v, g, 1, s_in=s)
    orr, sr = orc.recurrent(q, k, v, g, s_in=s)
    oT, sT = orc.chunkwise(q, k, v, g, 24, s_in=s)
    op, sp = orc.parallel(q, k, v, g, s_in=s)
    assert rel(o1, orr) < 1e-13 and rel(s1, sr) < 1e-13
    assert rel(oT, op) < 1e-13 and rel(sT, sp) < 1e-13


def test_chunkwise_rejects_chunk_not_dividing_T():
    q, k, v, _ = tiny(T=12)
    with pytest.raises(ValueError):
        orc.chunkwise(q, k, v, [0.9, 0.9], 5)


# ------------------------------------------------------------------ causality
@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunk8"])
def test_causality_future_tokens_do_not_change_the_past(form):
    """D[n][m] = 0 for m > n: perturbing tokens t >= t0 leaves every output
    before t0 bit-identical (jsqmd.com s3; aiqz.cc decay mask)."""
    q, k, v, s = tiny(seed=11, T=32)
    g = mi.gammas(2)
    t0 = 13
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rng = np.random.default_rng(1)
    for a in (q2, k2, v2):
        a[:, t0:] += rng.standard_normal(a[:, t0:].shape)
    run = {"parallel": orc.parallel, "recurrent": orc.recurrent,
           "chunk8": lambda *a, **kw: orc.chunkwise(*a[:4], 8, **kw)}[form]
    o1, _ = run(q, k, v, g, s_in=s)
    o2, _ = run(q2, k2, v2, g, s_in=s)
    assert np.array_equal(o1[:, :t0], o2[:, :t0])
    assert not np.allclose(o1[:, t0:], o2[:, t0:])


# -------------------------------------------------------------- closed forms
@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunk4"])
def test_all_ones_geometric_series(form):
    """No rotation, Q=K=V=1, zero state: O_raw[n][j] = s*dk*(1-g^(n+1))/(1-g)
    and S_out[i][j] = s*(1-g^T)/(1-g) (sum of the decay weights)."""
    B, T, H, dk, dv = 1, 16, 2, 4, 6
    g = np.array([0.9, 0.5], np.float32)
    ones = lambda d: np.ones((B, T, H, d))
    run = {"parallel": orc.parallel, "recurrent": orc.recurrent,
           "chunk4": lambda *a, **kw: orc.chunkwise(*a[:4], 4, **kw)}[form]
    o, s = run(ones(dk), ones(dk), ones(dv), g, rotate=False, groupnorm=False, scale=0.5)
    n = np.arange(T)
    for h in range(H):
        gh = np.float64(g[h])
        expect = 0.5 * dk * (1 - gh ** (n + 1)) / (1 - gh)
        assert np.allclose(o[0, :, h, :], expect[:, None], rtol=1e-13, atol=0)
        assert np.allclose(s[0, h], 0.5 * (1 - gh ** T) / (1 - gh), rtol=1e-13, atol=0)


def _complex_dot(qv, kv, n, m, theta, scale):
    """Re(sum_i qc_i e^{i n th_i} conj(kc_i e^{i m th_i})) * scale -- the
    complex-number reading of the rotation (jsqmd.com s2)."""
    qc = qv[0::2] + 1j * qv[1::2]
    kc = kv[0::2] + 1j * kv[1::2]
    return float(np.real(np.sum(qc * np.exp(1j * n * theta) * np.conj(kc * np.exp(1j * m * theta))))) * scale


@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunk8"])
def test_impulse_response(form):
    """K, V zero except token m0: O_raw[n] = g^(n-m0) (q~_n . k~_m0) v_m0 for
    n >= m0, else 0; the rotated dot product is evaluated with complex
    exponentials, independently of the oracle's real 2x2 rotation."""
    B, T, H, dk, dv = 1, 24, 1, 8, 5
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, T, H, dk))
    k = np.zeros((B, T, H, dk))
    v = np.zeros((B, T, H, dv))
    m0 = 9
    k[0, m0, 0] = rng.standard_normal(dk)
    v[0, m0, 0] = rng.standard_normal(dv)
    g = np.float32(0.8)
    theta = orc.default_theta(dk).astype(np.float64)
    scale = orc.default_scale(dk)
    run = {"parallel": orc.parallel, "recurrent": orc.recurrent,
           "chunk8": lambda *a, **kw: orc.chunkwise(*a[:4], 8, **kw)}[form]
    pos0 = 3
    o, _ = run(q, k, v, [g], groupnorm=False, pos0=pos0)
    for n in range(T):
        if n < m0:
            assert np.all(o[0, n, 0] == 0.0)
        else:
            w = np.float64(g) ** (n - m0) * _complex_dot(q[0, n, 0], k[0, m0, 0], pos0 + n,
                                                          pos0 + m0, theta, scale)
            assert np.allclose(o[0, n, 0], w * v[0, m0, 0], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ rotation
def test_rotation_sign_and_direction():
    """theta_shift = x cos + rotate_every_two(x) sin with rotate_every_two
    (x0, x1) -> (-x1, x0): e0 at angle 1 -> (cos 1, sin 1); e1 -> (-sin 1, cos 1)."""
    x = np.zeros((1, 2, 1, 2))
    x[0, :, 0, 0] = [1, 0]
    x[0, 1, 0] = [0, 1]
    x[0, 0, 0] = [1, 0]
    y = orc.rotate(x, theta=np.array([1.0], np.float32), pos0=1)
    assert np.allclose(y[0, 0, 0], [np.cos(1.0), np.sin(1.0)], rtol=0, atol=1e-15)
    y2 = orc.rotate(x, theta=np.array([1.0], np.float32), pos0=0)
    # token 1 sits at position 1 when pos0 = 0
    assert np.allclose(y2[0, 1, 0], [-np.sin(1.0), np.cos(1.0)], rtol=0, atol=1e-15)
    assert np.allclose(y2[0, 0, 0], [1, 0], rtol=0, atol=0)  # position 0: identity


def test_rotation_preserves_norm_and_relative_position():
    """Rotation is orthogonal per pair, and the rotated q . k depends only on
    the position difference (jsqmd.com s2: relative position kept)."""
    rng = np.random.default_rng(2)
    dk = 16
    x = rng.standard_normal((1, 40, 1, dk))
    y = orc.rotate(x, pos0=17)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    qv, kv = rng.standard_normal(dk), rng.standard_normal(dk)
    Q = np.tile(qv, (1, 40, 1, 1)).reshape(1, 40, 1, dk)
    Kt = np.tile(kv, (1, 40, 1, 1)).reshape(1, 40, 1, dk)
    for shift in (0, 5, 1000):
        qr = orc.rotate(Q, pos0=shift)[0, :, 0]
        kr = orc.rotate(Kt, pos0=shift)[0, :, 0]
        # q at position n+shift, k at position m+shift with n - m = 7
        d1 = qr[20] @ kr[13]
        d0 = orc.rotate(Q, pos0=0)[0, 20, 0] @ orc.rotate(Kt, pos0=0)[0, 13, 0]
        assert abs(d1 - d0) < 1e-12 * max(1.0, abs(d0))


def test_default_theta_and_scale():
    """theta_i = 10000^(-2i/dk); scale = dk^-0.5 (jsqmd.com s5: divide by sqrt(d))."""
    th = orc.default_theta(8)
    assert th.dtype == np.float32
    assert np.allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-7)
    assert orc.default_scale(256) == 0.0625


# ------------------------------------------------------------------ GroupNorm
def test_groupnorm_matches_torch_group_norm():
    """Per-head GroupNorm equals torch.nn.functional.group_norm (one group per
    head, no affine) in float64."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    B, T, H, dv = 2, 5, 3, 8
    x = rng.standard_normal((B, T, H, dv)) * 3 + 1
    y = orc.groupnorm(x, eps=1e-5)
    eps = float(np.float32(1e-5))
    ref = torch.nn.functional.group_norm(torch.from_numpy(x.reshape(B * T, H * dv)), H, eps=eps)
    assert np.allclose(y.reshape(B * T, H * dv), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_forms_apply_groupnorm_per_head_per_token():
    torch = pytest.importorskip("torch")
    q, k, v, s = tiny(seed=4, T=16)
    g = mi.gammas(2)
    raw, _ = orc.parallel(q, k, v, g, groupnorm=False, s_in=s)
    out, _ = orc.parallel(q, k, v, g, groupnorm=True, s_in=s)
    B, T, H, dv = raw.shape
    eps = float(np.float32(1e-5))
    ref = torch.nn.functional.group_norm(torch.from_numpy(raw.reshape(B * T, H * dv)), H, eps=eps)
    assert np.allclose(out.reshape(B * T, H * dv), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_groupnorm_scale_invariance():
    """GN(c x) = GN(x) up to eps (b99b.cn: GroupNorm's scale invariance)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 32))
    for c in (1e-2, 3.0, 1e3):
        assert rel(orc.groupnorm(c * x, eps=0.0), orc.groupnorm(x, eps=0.0)) < 1e-13
    y = orc.groupnorm(x)
    assert np.allclose(y.mean(-1), 0, atol=1e-14)


# ------------------------------------------- independent dense formulation
def test_parallel_matches_dense_mask_matrix_form():
    """O = (Q~ K~^T (.) D) V + diag(g^(n+1)) Q~ S_in with the n x n decay mask D
    built as a matrix (aiqz.cc 'parallel representation'), rotation done with
    complex exponentials; state = g^T S_in + K~^T diag(g^(T-1-m)) V."""
    B, T, H, dk, dv = 1, 20, 2, 6, 4
    q, k, v, s = tiny(seed=8, B=B, T=T, H=H, dk=dk, dv=dv)
    g = np.array([0.95, 0.7], np.float32)
    theta = orc.default_theta(dk).astype(np.float64)
    scale = orc.default_scale(dk)
    pos0 = 11
    o, so = orc.parallel(q, k, v, g, s_in=s, groupnorm=False, pos0=pos0)
    pos = pos0 + np.arange(T)
    for h in range(H):
        gh = np.float64(g[h])
        rot = np.exp(1j * pos[:, None] * theta[None, :])
        qc = (q[0, :, h, 0::2] + 1j * q[0, :, h, 1::2]) * rot
        kc = (k[0, :, h, 0::2] + 1j * k[0, :, h, 1::2]) * rot
        qr = np.stack([qc.real, qc.imag], -1).reshape(T, dk)
        kr = np.stack([kc.real, kc.imag], -1).reshape(T, dk) * scale
        n = np.arange(T)
        D = np.where(n[:, None] >= n[None, :], gh ** (n[:, None] - n[None, :]).clip(0), 0.0)
        ref = (qr @ kr.T * D) @ v[0, :, h] + (gh ** (n + 1))[:, None] * (qr @ s[0, h])
        assert rel(o[0, :, h], ref) < 1e-12
        sref = gh ** T * s[0, h] + kr.T @ (v[0, :, h] * (gh ** (T - 1 - n))[:, None])
        assert rel(so[0, h], sref) < 1e-12


# ------------------------------------------------------------- state hand-off
def test_state_handoff_is_associative():
    """The state replaces the KV cache (aiqz.cc 'engineering practice'):
    chunkwise over T1 then T2 (state handed over, positions continued) equals
    one pass over T1+T2; prefill then decode steps equal the parallel form."""
    q, k, v, s = tiny(seed=12, T=48)
    g = mi.gammas(2)
    T1 = 32
    o_all, s_all = orc.chunkwise(q, k, v, g, 16, s_in=s)
    o1, s1 = orc.chunkwise(q[:, :T1], k[:, :T1], v[:, :T1], g, 16, s_in=s)
    o2, s2 = orc.chunkwise(q[:, T1:], k[:, T1:], v[:, T1:], g, 8, s_in=s1, pos0=T1)
    assert rel(np.concatenate([o1, o2], 1), o_all) < 1e-12
    assert rel(s2, s_all) < 1e-12
    st = s1
    outs = []
    for t in range(T1, 48):
        ot, st = orc.step(q[:, t], k[:, t], v[:, t], st, g, pos=t)
        outs.append(ot)
    assert rel(np.stack(outs, 1), o_all[:, T1:]) < 1e-12
    assert rel(st, s_all) < 1e-12


def test_parallel_rows_match_full_parallel():
    q, k, v, s = tiny(seed=13, T=40)
    g = mi.gammas(2)
    o, _ = orc.parallel(q, k, v, g, s_in=s, pos0=2)
    rows = [0, 1, 17, 39]
    for h in range(2):
        r = orc.parallel_rows(q[0, :, h], k[0, :, h], v[0, :, h], g[h], rows, s_in=s[0, h], pos0=2)
        assert rel(r, o[0, rows, h]) < 1e-13


# ------------------------------------------------- row-normalised decay (option)
@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunk4"])
def test_row_normalised_decay_of_a_constant_sequence_is_one(form):
    """Q = K = V = 1, no rotation, scale 1/d_k, no GroupNorm: every score is 1
    and the raw output of the token at position p is the decay row sum
    sum_{j<=p} gamma^j, so the row-normalised output is exactly 1.  The
    second call continues the sequence at pos0 = 16 from the state the first
    call left (the state stands for the earlier positions), and must also
    give 1; counting only the call's own tokens would not."""
    B, T, H, dk, dv = 1, 16, 2, 4, 6
    g = np.array([0.9, 0.5], np.float32)
    ones = lambda d: np.ones((B, T, H, d))
    run = {"parallel": orc.parallel, "recurrent": orc.recurrent,
           "chunk4": lambda *a, **kw: orc.chunkwise(*a[:4], 4, **kw)}[form]
    kw = dict(rotate=False, groupnorm=False, scale=1.0 / dk, rownorm=True)
    o1, s1 = run(ones(dk), ones(dk), ones(dv), g, **kw)
    o2, _ = run(ones(dk), ones(dk), ones(dv), g, s_in=s1, pos0=T, **kw)
    assert np.allclose(o1, 1.0, rtol=1e-13, atol=0) and np.allclose(o2, 1.0, rtol=1e-13, atol=0)
    # closed form of the factor: the raw output times (1 - g)/(1 - g^(p+1))
    raw, _ = run(ones(dk), ones(dk), ones(dv), g, s_in=s1, pos0=T, rotate=False, groupnorm=False, scale=1.0 / dk)
    p = T + np.arange(T)
    for h in range(H):
        gh = np.float64(g[h])
        assert np.allclose(raw[0, :, h, 0], (1 - gh ** (p + 1)) / (1 - gh), rtol=1e-13, atol=0)


def test_row_normalised_decay_split_calls_equal_one_call():
    """A sequence split over two calls (state carried, positions continued)
    gives the same row-normalised outputs as one call."""
    q, k, v, s = tiny(seed=14, T=48)
    g = mi.gammas(2)
    T1 = 20
    kw = dict(rownorm=True, groupnorm=False)
    o_all, _ = orc.parallel(q, k, v, g, s_in=s, pos0=3, **kw)
    o1, s1 = orc.parallel(q[:, :T1], k[:, :T1], v[:, :T1], g, s_in=s, pos0=3, **kw)
    o2, _ = orc.chunkwise(q[:, T1:], k[:, T1:], v[:, T1:], g, 4, s_in=s1, pos0=3 + T1, **kw)
    assert rel(np.concatenate([o1, o2], 1), o_all) < 1e-12


def test_row_normalised_decay_under_groupnorm_moves_only_eps():
    """GroupNorm of x / r equals (x - mean) / sqrt(var + r^2 eps): with the
    raw outputs x and the row sums r, the normalised-decay output is
    GroupNorm with a per-row epsilon r^2 eps."""
    q, k, v, s = tiny(seed=15, T=24)
    g = np.array([0.9, 0.6], np.float32)
    eps = 1e-2
    raw, _ = orc.parallel(q, k, v, g, s_in=s, pos0=5, groupnorm=False)
    o, _ = orc.parallel(q, k, v, g, s_in=s, pos0=5, eps=eps, rownorm=True)
    p = 5 + np.arange(24)
    for h in range(2):
        gh = np.float64(g[h])
        r = (1 - gh ** (p + 1)) / (1 - gh)
        x = raw[0, :, h]
        mean = x.mean(-1, keepdims=True)
        var = ((x - mean) ** 2).mean(-1, keepdims=True)
        expect = (x - mean) / np.sqrt(var + (r ** 2)[:, None] * np.float64(np.float32(eps)))
        assert rel(o[0, :, h], expect) < 1e-12


# ------------------------------------------------------ Q/K/V projections
def test_projection_brute_force_and_identity():
    """The projection is the plain sum y[t][o] = sum_i x[t][i] w[o][i]:
    checked against explicit loops, and identity weights return x."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((2, 3, 5))
    w = rng.standard_normal((4, 5))
    y = orc.project(x, w)
    for b in range(2):
        for t in range(3):
            for o in range(4):
                assert abs(y[b, t, o] - sum(x[b, t, i] * w[o, i] for i in range(5))) < 1e-13
    assert np.array_equal(orc.project(x, np.eye(5)), x)
