"""GPU parity of the row-normalised decay option (MSR_FLAG_DECAY_ROWNORM):
each output row divided by the sum of its decay weights over every absolute
position 0 .. p, before GroupNorm.  Covers the chunkwise and parallel forms
on the MFMA and general paths (incoming state, start positions, with and
without GroupNorm), the decode step, multi-token calls and the backward
pass, against the fp64 oracle.  GroupNorm sees the factor only through eps,
so the GroupNorm cases use eps = 1e-2, where it shows.
Tolerance as in the other parity tests: 1e-4 (fp32), 2e-2 (bf16)."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import grad as og
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu


def _msr():
    import retnet_scale_retention_amd as msr
    return msr


# (name, B, T, H, dk, dv, dtype, chunk)
CASES = [
    ("f32-general", 1, 64, 2, 16, 16, "f32", 16),
    ("bf16-mfma-b64", 2, 256, 2, 64, 128, "bf16", 64),
    ("bf16-mfma-dk256-b128", 1, 256, 2, 256, 512, "bf16", 128),  # d_v over 8 slices: statistics + finalize
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("form", ["chunkwise", "parallel"])
@pytest.mark.parametrize("groupnorm", [False, True])
@pytest.mark.parametrize("pos0", [0, 3, 900])
def test_rownorm_forms_vs_oracle(case, form, groupnorm, pos0):
    name, B, T, H, dk, dv, dtype, chunk = case
    torch, dev = torch_dev()
    msr = _msr()
    w = mi.Workload("rownorm-" + name, 60, B, T, H, dk, dv, dtype, (chunk,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s_in = mi.state(w, 0.5) if pos0 else None
    eps = 1e-2 if groupnorm else 1e-5
    ro, rs = orc.parallel(q, k, v, g, s_in=s_in, pos0=pos0, eps=eps, groupnorm=groupnorm, rownorm=True)
    flags = msr.MSR_FLAG_DECAY_ROWNORM | (0 if groupnorm else msr.MSR_FLAG_NO_GROUPNORM)
    qd, kd, vd = (up(x, dtype, dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    note(f"{name} {form} gn={groupnorm} pos0={pos0}")
    if form == "chunkwise":
        o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, pos0=pos0, eps=eps, flags=flags)
    else:
        o, s = msr.msr_parallel(qd, kd, vd, g, state_in=sd, pos0=pos0, eps=eps, flags=flags)
    torch.cuda.synchronize()
    eo, es = out_err(down(o), ro), state_err(down(s), rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


def test_rownorm_row_positions_vs_oracle():
    torch, dev = torch_dev()
    msr = _msr()
    B, T, H, dk, dv = 2, 256, 2, 64, 128
    w = mi.Workload("rownorm-rows", 61, B, T, H, dk, dv, "bf16", (64,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s_in = mi.state(w, 0.5)
    pos = np.array([0, 700], np.int64)
    ro = np.concatenate([orc.parallel(q[b:b + 1], k[b:b + 1], v[b:b + 1], g, s_in=s_in[b:b + 1], pos0=int(pos[b]),
                                      groupnorm=False, rownorm=True)[0] for b in range(B)])
    o, _ = msr.msr_chunkwise(*(up(x, "bf16", dev) for x in (q, k, v)), g, 64, state_in=torch.from_numpy(s_in).to(dev),
                             pos_rows=torch.from_numpy(pos).to(dev),
                             flags=msr.MSR_FLAG_DECAY_ROWNORM | msr.MSR_FLAG_NO_GROUPNORM)
    torch.cuda.synchronize()
    eo = out_err(down(o), ro)
    note(f"rows {pos.tolist()}: O err {eo:.2e}")
    assert eo < TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ntok", [1, 4])
def test_rownorm_decode_vs_oracle(dtype, ntok):
    """Steps of 1 token (msr_recurrent_step) or calls of 4 tokens with the
    state carried in place, from position 50 on."""
    torch, dev = torch_dev()
    msr = _msr()
    B, H, dk, dv, P = 3, 2, 64, 128, 50
    w = mi.Workload("rownorm-dec", 62, B, 8, H, dk, dv, dtype, (8,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s0 = mi.state(w, 0.5)
    ro, rs = orc.parallel(q, k, v, g, s_in=s0, pos0=P, groupnorm=False, rownorm=True)
    qd, kd, vd = (up(x, dtype, dev) for x in (q, k, v))
    st = torch.from_numpy(s0).to(dev)
    flags = msr.MSR_FLAG_DECAY_ROWNORM | msr.MSR_FLAG_NO_GROUPNORM
    outs = []
    for t0 in range(0, 8, ntok):
        if ntok == 1:
            outs.append(msr.msr_recurrent_step(qd[:, t0].contiguous(), kd[:, t0].contiguous(), vd[:, t0].contiguous(), st,
                                                  g, P + t0, flags=flags)[:, None])
        else:
            sl = slice(t0, t0 + ntok)
            o, _ = msr.msr_chunkwise(qd[:, sl].contiguous(), kd[:, sl].contiguous(), vd[:, sl].contiguous(), g, ntok,
                                     state_in=st, state_out=st,
                                     pos0=P + t0, flags=flags)
            outs.append(o)
    torch.cuda.synchronize()
    eo = out_err(down(torch.cat(outs, 1)), ro)
    es = state_err(down(st), rs)
    note(f"decode {dtype} {ntok} tok/call: O err {eo:.2e} state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


# (name, B, T, H, dk, dv, dtype, chunk)
BWD = [("f32-general", 1, 64, 2, 16, 16, "f32", 16), ("bf16-mfma", 2, 256, 2, 64, 128, "bf16", 64)]


@pytest.mark.parametrize("case", BWD, ids=[c[0] for c in BWD])
@pytest.mark.parametrize("groupnorm", [False, True])
def test_rownorm_backward_vs_oracle(case, groupnorm):
    name, B, T, H, dk, dv, dtype, chunk = case
    torch, dev = torch_dev()
    msr = _msr()
    w = mi.Workload("rownorm-bwd-" + name, 63, B, T, H, dk, dv, dtype, (chunk,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    rng = np.random.default_rng(64)
    do = mi.quantize(rng.standard_normal((B, T, H, dv)).astype(np.float32), dtype)
    ds = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    s_in = mi.state(w, 0.5)
    eps = 1e-2 if groupnorm else 1e-5
    ref = og.backward(q, k, v, g, do, grad_state=ds, s_in=s_in, pos0=3, eps=eps, groupnorm=groupnorm,
                      rownorm=True)
    flags = msr.MSR_FLAG_DECAY_ROWNORM | (0 if groupnorm else msr.MSR_FLAG_NO_GROUPNORM)
    t = lambda x: torch.from_numpy(x).to(dev)
    got = msr.msr_chunkwise_backward(*(up(x, dtype, dev) for x in (q, k, v)), g, chunk, up(do, dtype, dev),
                                     grad_state=t(ds), state_in=t(s_in), pos0=3, eps=eps, flags=flags)
    torch.cuda.synchronize()
    errs = [out_err(down(got[i]), ref[i]) for i in range(3)] + [state_err(down(got[3]), ref[3])]
    note(f"backward {name} gn={groupnorm}: " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) < TOL[dtype]
