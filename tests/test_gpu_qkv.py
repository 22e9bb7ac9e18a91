"""GPU parity of the Q/K/V projections in front of retention
(msr_qkv_projection: a bf16 MFMA GEMM with the rotation and K's scale in its
epilogue) and of the composite msr_qkv_chunkwise (projections, then the
chunkwise form), against the fp64 oracle: the projection as a float64
matrix product, the rotation and the forms from oracle/oracle.py.
Inputs: X ~ N(0, 1), weights ~ N(0, 1/d_model), both bf16.
Tolerance: 2e-2 (bf16), max relative error per (batch, head) slice."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev

pytestmark = pytest.mark.gpu


def _msr():
    import retnet_scale_retention_amd as msr
    return msr


def make(seed, B, T, dm, H, dk, dv):
    rng = np.random.default_rng(seed)
    x = mi.round_bf16(rng.standard_normal((B, T, dm)).astype(np.float32))
    w = [mi.round_bf16((rng.standard_normal((H * d, dm)) / np.sqrt(dm)).astype(np.float32)) for d in (dk, dk, dv)]
    return x, w


def oracle_qkv(x, w, H, dk, dv, pos, rotate=True, scale=None):
    """Projections, then the rotation (and K's scale) per batch row at its start position."""
    B, T, _ = x.shape
    q, k, v = (orc.project(x, wi).reshape(B, T, H, -1) for wi in w)
    if rotate:
        sc = float(np.float32(1 / np.sqrt(dk))) if scale is None else scale
        q = np.concatenate([orc.rotate(q[b:b + 1], pos0=int(pos[b])) for b in range(B)])
        k = np.concatenate([orc.rotate(k[b:b + 1], pos0=int(pos[b]), factor=sc) for b in range(B)])
    return q, k, v


def dev_bf16(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)


# (name, B, T, d_model, H, dk, dv)
PROJ = [
    ("M200-ragged", 2, 100, 128, 2, 64, 128),      # 200 tokens: a partial 128-row tile
    ("N192", 1, 256, 256, 3, 64, 64),              # 192 features: a partial 128-column tile
    ("dk256-dv512", 1, 130, 512, 2, 256, 512),
    ("tiny", 1, 5, 64, 1, 8, 4),
]


@pytest.mark.parametrize("case", PROJ, ids=[c[0] for c in PROJ])
@pytest.mark.parametrize("mode", ["rotate", "plain", "rows"])
def test_projection_vs_oracle(case, mode):
    name, B, T, dm, H, dk, dv = case
    torch, dev = torch_dev()
    msr = _msr()
    x, w = make(70, B, T, dm, H, dk, dv)
    pos = np.array([5, 9000][:B] if mode == "rows" else [5] * B, np.int64)
    rq, rk, rv = oracle_qkv(x, w, H, dk, dv, pos, rotate=mode != "plain")
    xd = dev_bf16(torch, dev, x)
    wd = [dev_bf16(torch, dev, wi) for wi in w]
    kw = dict(pos0=5)
    if mode == "plain":
        kw["flags"] = msr.MSR_FLAG_NO_ROTATE
    if mode == "rows":
        kw["pos_rows"] = torch.from_numpy(pos).to(dev)
    note(f"{name} {mode}")
    q, k, v = msr.msr_qkv_projection(xd, *wd, H, **kw)
    torch.cuda.synchronize()
    errs = [out_err(down(q), rq), out_err(down(k), rk), out_err(down(v), rv)]
    note("  errs " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) < TOL["bf16"]


def test_projection_7b_shape_sampled_rows():
    """The 7B-shaped layer (B=2, T=8192, d_model=4096, H=16, d_k=256,
    d_v=512), as the bench runs it; 48 sampled tokens against the oracle."""
    torch, dev = torch_dev()
    msr = _msr()
    B, T, dm, H, dk, dv = 2, 8192, 4096, 16, 256, 512
    x = mi.device_normal((B, T, dm), 7001, dev, torch.bfloat16)
    wq = (mi.device_normal((H * dk, dm), 7002, dev, torch.float32) / np.sqrt(dm)).to(torch.bfloat16)
    wk = (mi.device_normal((H * dk, dm), 7003, dev, torch.float32) / np.sqrt(dm)).to(torch.bfloat16)
    wv = (mi.device_normal((H * dv, dm), 7004, dev, torch.float32) / np.sqrt(dm)).to(torch.bfloat16)
    q, k, v = msr.msr_qkv_projection(x, wq, wk, wv, H, pos0=0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(71)
    rows = [(int(b), int(t)) for b, t in zip(rng.integers(0, B, 48), rng.integers(0, T, 48))] + [(0, 0), (1, T - 1)]
    xs = np.stack([down(x[b, t]) for b, t in rows])[None]            # [1, R, dm]
    w = [down(wi) for wi in (wq, wk, wv)]
    sc = float(np.float32(1 / np.sqrt(dk)))
    worst = 0.0
    for i, (b, t) in enumerate(rows):
        yq, yk, yv = (orc.project(xs[:, i:i + 1], wi).reshape(1, 1, H, -1) for wi in w)
        yq, yk = orc.rotate(yq, pos0=t), orc.rotate(yk, pos0=t, factor=sc)
        for got, ref in ((q[b, t], yq[0, 0]), (k[b, t], yk[0, 0]), (v[b, t], yv[0, 0])):
            g = down(got)
            worst = max(worst, float(np.max(np.abs(g - ref) / np.max(np.abs(ref), axis=1, keepdims=True))))
    note(f"7b projection, {len(rows)} tokens: max rel err {worst:.2e}")
    assert worst < TOL["bf16"]


# (name, B, T, d_model, H, dk, dv, chunk)
LAYER = [
    ("mfma-b64", 2, 256, 128, 2, 64, 128, 64),
    ("mfma-b128-dk256", 1, 256, 256, 2, 256, 512, 128),
    ("general-T100", 1, 100, 64, 2, 32, 32, 64),   # last chunk shorter than b
]


@pytest.mark.parametrize("case", LAYER, ids=[c[0] for c in LAYER])
@pytest.mark.parametrize("with_state", [False, True])
def test_qkv_chunkwise_vs_oracle(case, with_state):
    name, B, T, dm, H, dk, dv, chunk = case
    torch, dev = torch_dev()
    msr = _msr()
    x, w = make(72, B, T, dm, H, dk, dv)
    g = mi.gammas(H)
    rng = np.random.default_rng(73)
    s_in = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32) if with_state else None
    q, k, v = (orc.project(x, wi).reshape(B, T, H, -1) for wi in w)
    ro, rs = orc.parallel(q, k, v, g, s_in=s_in, pos0=7)
    xd = dev_bf16(torch, dev, x)
    wd = [dev_bf16(torch, dev, wi) for wi in w]
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    o, s = msr.msr_qkv_chunkwise(xd, *wd, g, chunk, state_in=sd, pos0=7)
    torch.cuda.synchronize()
    eo, es = out_err(down(o), ro), state_err(down(s), rs)
    note(f"{name} state={with_state}: O err {eo:.2e} state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
