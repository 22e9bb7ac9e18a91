"""GPU parity: every form of libmsr.so (called through the C ABI) against
the fp64 oracle on the same seeded inputs, element by element.
Tolerance (max relative error per (batch, head) slice): 1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 accumulation."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu


def _msr():
    import retnet_scale_retention_amd as msr
    return msr


def run_gpu(form, q, k, v, g, dtype, chunk=None, s_in=None, **kw):
    torch, dev = torch_dev()
    msr = _msr()
    qd, kd, vd = (up(x, dtype, dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(np.ascontiguousarray(s_in, np.float32)).to(dev)
    if form == "parallel":
        o, s = msr.msr_parallel(qd, kd, vd, g, state_in=sd, **kw)
    else:
        o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, **kw)
    torch.cuda.synchronize()
    return down(o), down(s)


def run_steps(q, k, v, g, dtype, s_in, pos0, **kw):
    """Recurrent form on the GPU: one msr_recurrent_step per token."""
    torch, dev = torch_dev()
    msr = _msr()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    st = (torch.zeros((B, H, dk, dv), dtype=torch.float32, device=dev) if s_in is None
          else torch.from_numpy(np.ascontiguousarray(s_in, np.float32)).to(dev))
    outs = []
    for t in range(T):
        o = msr.msr_recurrent_step(up(q[:, t], dtype, dev).contiguous(), up(k[:, t], dtype, dev).contiguous(),
                                   up(v[:, t], dtype, dev).contiguous(), st, g, pos0 + t, **kw)
        outs.append(down(o))
    torch.cuda.synchronize()
    return np.stack(outs, 1), down(st)


# ------------------------------------------------------------ tiny (fp32)
TINY = mi.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny_inputs():
    q, k, v = mi.qkv(TINY)
    s = mi.state(TINY, 0.5)
    return q, k, v, s


@pytest.mark.parametrize("with_state", [False, True])
def test_tiny_all_forms_vs_oracle(tiny_inputs, with_state):
    q, k, v, s = tiny_inputs
    s_in = s if with_state else None
    g = mi.gammas(TINY.H)
    ro, rs = orc.parallel(q, k, v, g, s_in=s_in)
    note("tiny: parallel")
    o, st = run_gpu("parallel", q, k, v, g, "f32", s_in=s_in)
    assert out_err(o, ro) < TOL["f32"] and state_err(st, rs) < TOL["f32"]
    forms = {"parallel": o}
    for b in TINY.chunks:
        note(f"tiny: chunkwise b={b}")
        oc, sc = run_gpu("chunk", q, k, v, g, "f32", chunk=b, s_in=s_in)
        assert out_err(oc, ro) < TOL["f32"], b
        assert state_err(sc, rs) < TOL["f32"], b
        forms[f"chunk{b}"] = oc
    note("tiny: recurrent steps")
    orr, sr = run_steps(q, k, v, g, "f32", s_in, 0)
    assert out_err(orr, ro) < TOL["f32"] and state_err(sr, rs) < TOL["f32"]
    forms["recurrent"] = orr
    names = list(forms)
    for a in names:  # the GPU's own forms cross-check
        for b2 in names:
            assert out_err(forms[a], forms[b2]) < TOL["f32"], (a, b2)


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_tiny_flags(tiny_inputs, flags):
    q, k, v, s = tiny_inputs
    g = mi.gammas(TINY.H)
    ro, rs = orc.chunkwise(q, k, v, g, 16, s_in=s, rotate=not (flags & 1), groupnorm=not (flags & 2))
    note(f"tiny: flags={flags}")
    o, st = run_gpu("chunk", q, k, v, g, "f32", chunk=16, s_in=s, flags=flags)
    assert out_err(o, ro) < TOL["f32"] and state_err(st, rs) < TOL["f32"]


def test_tiny_explicit_theta_scale_eps_pos0(tiny_inputs):
    q, k, v, s = tiny_inputs
    g = np.array([0.5, 1.0], np.float32)  # gamma = 1 is allowed (no decay)
    theta = np.linspace(0.9, 0.001, TINY.dk // 2).astype(np.float32)
    kw = dict(theta=theta, scale=0.3, eps=1e-3, pos0=123457)
    ro, rs = orc.parallel(q, k, v, g, s_in=s, **kw)
    note("tiny: explicit parameters")
    o, st = run_gpu("chunk", q, k, v, g, "f32", chunk=16, s_in=s, **kw)
    assert out_err(o, ro) < TOL["f32"] and state_err(st, rs) < TOL["f32"]
    o2, st2 = run_gpu("parallel", q, k, v, g, "f32", s_in=s, **kw)
    assert out_err(o2, ro) < TOL["f32"] and state_err(st2, rs) < TOL["f32"]


def test_state_out_may_alias_state_in(tiny_inputs):
    torch, dev = torch_dev()
    msr = _msr()
    q, k, v, s = tiny_inputs
    g = mi.gammas(TINY.H)
    ro, rs = orc.parallel(q, k, v, g, s_in=s)
    for form in ("parallel", "chunk"):
        note(f"alias: {form}")
        sd = torch.from_numpy(s).to(dev)
        qd, kd, vd = (up(x, "f32", dev) for x in (q, k, v))
        if form == "parallel":
            o, _ = msr.msr_parallel(qd, kd, vd, g, state_in=sd, state_out=sd)
        else:
            o, _ = msr.msr_chunkwise(qd, kd, vd, g, 16, state_in=sd, state_out=sd)
        torch.cuda.synchronize()
        assert out_err(down(o), ro) < TOL["f32"]
        assert state_err(down(sd), rs) < TOL["f32"]


def test_empty_inputs():
    torch, dev = torch_dev()
    msr = _msr()
    g = mi.gammas(2)
    s = mi.state(TINY)[:1]
    sd = torch.from_numpy(s).to(dev)
    z = torch.zeros((1, 0, 2, 16), device=dev)
    note("empty: T=0")
    o, so = msr.msr_chunkwise(z, z, z, g, 4, state_in=sd)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 16) and np.array_equal(down(so), s.astype(np.float64))
    o, so = msr.msr_parallel(z, z, z, g)
    torch.cuda.synchronize()
    assert np.all(down(so) == 0)
    zb = torch.zeros((0, 8, 2, 16), device=dev)
    o, so = msr.msr_chunkwise(zb, zb, zb, g, 4)
    torch.cuda.synchronize()
    assert o.shape == (0, 8, 2, 16)


# ------------------------------------------------------------ decode step
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_vs_oracle(dtype):
    w = mi.Workload("dec-test", 11, 3, 6, 4, 64, 128, dtype, (1,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.1)
    g = mi.gammas(w.H)
    pos0 = 2047
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=pos0)
    note(f"decode steps {dtype}")
    o, st = run_steps(q, k, v, g, dtype, s, pos0)
    assert out_err(o, ro) < TOL[dtype]
    assert state_err(st, rs) < 1e-5  # the state is fp32 in both precisions


@pytest.mark.parametrize("dv", [4, 16, 1024])
def test_decode_shapes(dv):
    w = mi.Workload("dec-shape", 12, 2, 2, 3, 8, dv, "f32", (1,))
    q, k, v = mi.qkv(w)
    s = mi.state(w)
    g = mi.gammas(w.H)
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=5)
    note(f"decode dv={dv}")
    o, st = run_steps(q, k, v, g, "f32", s, 5)
    assert out_err(o, ro) < TOL["f32"] and state_err(st, rs) < TOL["f32"]


# ------------------------------------------------- ragged / odd shapes
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 45, 3, 6, 12, 15), (1, 40, 2, 34, 20, 8), (1, 96, 1, 2, 4, 32)])
def test_odd_shapes(dtype, shape):
    B, T, H, dk, dv, b = shape
    w = mi.Workload("odd", 13, B, T, H, dk, dv, dtype, (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.2)
    g = mi.gammas(H)
    ro, rs = orc.parallel(q, k, v, g, s_in=s, pos0=7)
    note(f"odd shape {shape} {dtype}")
    o, st = run_gpu("chunk", q, k, v, g, dtype, chunk=b, s_in=s, pos0=7)
    assert out_err(o, ro) < TOL[dtype] and state_err(st, rs) < TOL[dtype]
    o2, st2 = run_gpu("parallel", q, k, v, g, dtype, s_in=s, pos0=7)
    assert out_err(o2, ro) < TOL[dtype] and state_err(st2, rs) < TOL[dtype]


# ------------------------------------------------------- small model layer
SMALL = mi.WORKLOADS["small"]


def test_small_layer_chunkwise_and_parallel():
    q, k, v = mi.qkv(SMALL)
    g = mi.gammas(SMALL.H)
    b = SMALL.chunks[0]
    note("small: oracle")
    ro, rs = orc.chunkwise(q, k, v, g, b)
    note("small: gpu chunkwise")
    o, st = run_gpu("chunk", q, k, v, g, "bf16", chunk=b)
    assert out_err(o, ro) < TOL["bf16"] and state_err(st, rs) < TOL["bf16"]
    note("small: gpu parallel")
    o2, st2 = run_gpu("parallel", q, k, v, g, "bf16")
    assert out_err(o2, ro) < TOL["bf16"] and state_err(st2, rs) < TOL["bf16"]
    assert out_err(o2, o) < TOL["bf16"]


# ------------------------------------------- rotation at large positions
BIG_POS = 3_000_000_017  # angles of 3e9 rad and more: the fp64 angle reduction


@pytest.mark.parametrize("route", ["mfma-chunk", "mfma-parallel", "generic-fp32", "steps-fp32", "steps-bf16"])
def test_large_start_position(route):
    """Every rotating kernel at a start position near 3e9 (explicit fp32 theta on
    both sides, so that both rotate by the same frequencies)."""
    dtype = "f32" if route.endswith("fp32") else "bf16"
    dk, dv = (256, 256) if route.startswith("mfma") else (32, 32)
    T = 256 if route.startswith("mfma") else 24
    w = mi.Workload("bigpos", 71, 1, T, 2, dk, dv, dtype, (128,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(2)
    th = orc.default_theta(dk)
    if route == "mfma-parallel":
        ro, rs = orc.parallel(q, k, v, g, s_in=s, pos0=BIG_POS, theta=th)
        o, st = run_gpu("parallel", q, k, v, g, dtype, s_in=s, pos0=BIG_POS, theta=th)
    elif route.startswith("steps"):
        ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=BIG_POS, theta=th)
        o, st = run_steps(q, k, v, g, dtype, s, BIG_POS, theta=th)
    else:
        chunk = 128 if route == "mfma-chunk" else 8
        ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=BIG_POS, theta=th)
        o, st = run_gpu("chunk", q, k, v, g, dtype, chunk=chunk, s_in=s, pos0=BIG_POS, theta=th)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"{route} pos0 {BIG_POS}: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
