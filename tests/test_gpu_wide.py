"""GPU parity of the wide-slice chunk kernel (a workgroup per 256 value
columns; taken for d_k 128 or 256 and d_v a multiple of 256, at chunk 64, and at
chunk 128 when no segments are needed)
against the fp64 oracle: one segment and several, an incoming state, a
non-zero start position, gammas that rescale the carried state every chunk
or never, the flags, an outgoing state written over the incoming one, and
run-to-run determinism.  Tolerance 2e-2 (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu

CASES = [  # (B, T, H, dk, dv, chunk); segments per pair in the comment
    (1, 512, 2, 128, 256, 64),     # 4
    (2, 320, 4, 128, 256, 64),     # 1 (5 chunks)
    (1, 1024, 2, 256, 256, 64),    # 8
    (1, 384, 2, 256, 512, 64),     # 2
    (2, 1024, 1, 256, 512, 64),    # 8
]
GAMMAS = np.array([0.75, 0.96875, 0.999, 1.0], dtype=np.float32)


def run(q, k, v, g, chunk, s_in=None, **kw):
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, **kw)
    torch.cuda.synchronize()
    return down(o), down(s)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_wide_vs_oracle(case):
    B, T, H, dk, dv, b = case
    w = mi.Workload("wide", 41, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    for g in (mi.gammas(H), np.resize(GAMMAS, H).astype(np.float32)):
        note(f"wide {case} gamma {g}: oracle")
        ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=5)
        note(f"wide {case}: gpu")
        o, st = run(q, k, v, g, b, s_in=s, pos0=5)
        eo, es = out_err(o, ro), state_err(st, rs)
        note(f"  O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("flags", [1, 2, 4])  # no rotation / no GroupNorm / row-normalised decay
def test_wide_flags(flags):
    w = mi.Workload("wide-flags", 42, 1, 1024, 2, 256, 256, "bf16", (64,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(2)
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=7, rotate=not (flags & 1), groupnorm=not (flags & 2),
                           rownorm=bool(flags & 4))
    note(f"wide flags {flags}")
    o, st = run(q, k, v, g, 64, s_in=s, pos0=7, flags=flags)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_wide_state_out_over_state_in_and_determinism():
    """With segments, the outgoing state may overwrite the incoming one (the
    full pass reads a copy the state-only pass set aside); two runs agree
    bit for bit."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.Workload("wide-alias", 43, 1, 1024, 2, 256, 512, "bf16", (64,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(2)
    ro, rs = orc.recurrent(q, k, v, g, s_in=s)
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = torch.from_numpy(s).to(dev)
    note("wide alias")
    o, s2 = msr.msr_chunkwise(qd, kd, vd, g, 64, state_in=sd, state_out=sd)
    torch.cuda.synchronize()
    assert s2.data_ptr() == sd.data_ptr()
    assert out_err(down(o), ro) < TOL["bf16"] and state_err(down(sd), rs) < TOL["bf16"]
    o1, s1 = run(q, k, v, g, 64, s_in=s)
    o2, s2b = run(q, k, v, g, 64, s_in=s)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2b)
    assert out_err(o1, ro) < TOL["bf16"] and state_err(s1, rs) < TOL["bf16"]


@pytest.mark.parametrize("gamma", [0.5, 0.25])
def test_wide_split_scores_strong_decay(gamma):
    """The split-scores option (two-term bf16 q~, k~ in the scores) on the
    wide-slice kernel: within tolerance at strong decay and no worse than the
    plain call."""
    import retnet_scale_retention_amd as msr
    w = mi.Workload("wide-strong", 44, 1, 512, 2, 256, 512, "bf16", (64,))
    q, k, v = mi.qkv(w)
    g = np.full(2, gamma, np.float32)
    s = mi.state(w, 0.5)
    ro, rs = orc.chunkwise(q, k, v, g, 64, s_in=s, pos0=9)
    note(f"wide split scores gamma {gamma}")
    o1, s1 = run(q, k, v, g, 64, s_in=s, pos0=9)
    o2, s2 = run(q, k, v, g, 64, s_in=s, pos0=9, flags=msr.MSR_FLAG_SPLIT_SCORES)
    e1, e2 = out_err(o1, ro), out_err(o2, ro)
    note(f"  O err {e1:.2e} plain, {e2:.2e} split scores; state err {state_err(s2, rs):.2e}")
    assert e2 < TOL["bf16"] and state_err(s2, rs) < TOL["bf16"]
    assert e2 <= e1 * 1.05


# b = 128 takes the wide-slice kernel when one workgroup per (pair, 256
# columns) already fills the GPU, i.e. with no segments
CASES_128 = [  # (B, T, H, dk, dv, chunk)
    (8, 256, 16, 256, 256, 128),
    (4, 384, 32, 128, 256, 128),
]


@pytest.mark.parametrize("case", CASES_128, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_wide_b128_vs_oracle(case):
    B, T, H, dk, dv, b = case
    w = mi.Workload("wide128", 45, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = np.resize(GAMMAS, H).astype(np.float32)
    note(f"wide b=128 {case}: oracle")
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=5)
    o, st = run(q, k, v, g, b, s_in=s, pos0=5)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
