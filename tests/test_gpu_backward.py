"""GPU parity of the backward pass (msr_chunkwise_backward) against the
oracle's gradients (oracle/grad.py: the parallel definition in float64,
differentiated by autograd; pinned to finite differences of the C oracle).
Loss L = sum(O * dO) + sum(S_out * dS_out).  Tolerance as for the forward:
max relative error per (batch, head) slice 1e-4 for fp32 inputs, 2e-2 for
bf16 inputs (gradients returned in bf16)."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import grad as og
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu

# (name, B, T, H, dk, dv, dtype, chunk)
CASES = [
    ("f32-tiny", 1, 64, 2, 16, 16, "f32", 16),
    ("f32-T50-b16", 2, 50, 2, 16, 32, "f32", 16),   # last chunk shorter than b
    ("bf16-small", 2, 256, 2, 64, 128, "bf16", 64),
    ("bf16-dk128", 1, 128, 2, 128, 64, "bf16", 128),
    ("bf16-dv512", 1, 256, 2, 64, 512, "bf16", 64),    # d_v in two parts of 256 on the MFMA path
    ("bf16-dv320", 1, 128, 1, 128, 320, "bf16", 64),   # parts 256 + 64
    ("bf16-dv448", 1, 128, 2, 64, 448, "bf16", 64),    # three parts: 256 + 128 + 64
    ("bf16-T200", 1, 200, 2, 64, 128, "bf16", 64),     # b not dividing T: general path
]


def run(case, with_state, grad_state, flags=0, pos_rows=None, seed=50):
    name, B, T, H, dk, dv, dtype, chunk = case
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.Workload("bwd-" + name, seed, B, T, H, dk, dv, dtype, (chunk,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    rng = np.random.default_rng(seed + 1)
    do = mi.quantize(rng.standard_normal((B, T, H, dv)).astype(np.float32), dtype)
    ds = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if grad_state else None
    s_in = mi.state(w, 0.5) if with_state else None
    kw = dict(rotate=not (flags & 1), groupnorm=not (flags & 2))
    if pos_rows is not None:
        kw["pos_rows"] = pos_rows
    else:
        kw["pos0"] = 3
    ref = og.backward(q, k, v, g, do, grad_state=ds, s_in=s_in, **kw)
    qd, kd, vd, dod = (up(x, dtype, dev) for x in (q, k, v, do))
    t = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    pr = None if pos_rows is None else torch.tensor(pos_rows, dtype=torch.int64, device=dev)
    got = msr.msr_chunkwise_backward(qd, kd, vd, g, chunk, dod, grad_state=t(ds), state_in=t(s_in),
                                     flags=flags, pos0=3, pos_rows=pr)
    torch.cuda.synchronize()
    errs = [out_err(down(got[0]), ref[0]), out_err(down(got[1]), ref[1]), out_err(down(got[2]), ref[2]),
            state_err(down(got[3]), ref[3])]
    note(f"{name} state={with_state} dS={grad_state} flags={flags}: dQ {errs[0]:.2e} dK {errs[1]:.2e} "
         f"dV {errs[2]:.2e} dS_in {errs[3]:.2e}")
    return errs, TOL[dtype]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("with_state,grad_state", [(False, False), (True, True)])
def test_backward_vs_oracle(case, with_state, grad_state):
    errs, tol = run(case, with_state, grad_state)
    assert max(errs) < tol


@pytest.mark.parametrize("flags", [1, 2, 3])  # no rotation / no GroupNorm / neither
@pytest.mark.parametrize("case", [CASES[0], CASES[2]], ids=["f32-general", "bf16-mfma"])
def test_backward_flags_vs_oracle(case, flags):
    errs, tol = run(case, True, True, flags=flags)
    assert max(errs) < tol


def test_backward_row_positions_vs_oracle():
    errs, tol = run(CASES[2], True, False, pos_rows=[5, 700])
    assert max(errs) < tol


@pytest.mark.parametrize("seed", [51, 52, 53])
@pytest.mark.parametrize("case", [CASES[2], CASES[3]], ids=["bf16-small", "bf16-dk128"])
def test_backward_no_state_seeds(case, seed):
    """Zero incoming state: the first tokens' pre-norm outputs are built from
    few keys, where the gradients are most sensitive to score rounding."""
    errs, tol = run(case, False, False, seed=seed)
    assert max(errs) < tol


def test_backward_7b_shape_sampled_pairs():
    """The 7B-shaped backward (B=2, T=8192, H=16, d_k=256, d_v=512, b=128,
    bf16, dS_out given) in the launch configuration the bench times; the
    (batch, head) pairs are independent, so the oracle recomputes two of them
    alone at full length."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    B, T, H, dk, dv, chunk = 2, 8192, 16, 256, 512, 128
    shp = lambda d: (B, T, H, d)
    q = mi.device_normal(shp(dk), 4001, dev, torch.bfloat16)
    k = mi.device_normal(shp(dk), 4002, dev, torch.bfloat16)
    v = mi.device_normal(shp(dv), 4003, dev, torch.bfloat16)
    do = mi.device_normal(shp(dv), 4004, dev, torch.bfloat16)
    ds = mi.device_normal((B, H, dk, dv), 4005, dev, torch.float32)
    g = mi.gammas(H)
    got = msr.msr_chunkwise_backward(q, k, v, g, chunk, do, grad_state=ds)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 13)):
        sl = lambda t: down(t[b:b + 1, :, h:h + 1])
        ref = og.backward(sl(q), sl(k), sl(v), g[h:h + 1], sl(do), grad_state=down(ds[b:b + 1, h:h + 1]))
        errs = [out_err(sl(got[i]), ref[i]) for i in range(3)] + [state_err(down(got[3][b:b + 1, h:h + 1]), ref[3])]
        note(f"7b backward pair (b={b}, h={h}): " + " ".join(f"{e:.2e}" for e in errs))
        assert max(errs) < TOL["bf16"]
