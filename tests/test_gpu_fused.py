"""GPU parity of the fused schedule of the chunkwise form (MSR_FLAG_FUSED:
rotation, intra-chunk scores and, at d_v = 256, GroupNorm inside the
recurrence workgroups, from the caller's Q, K, V) against the fp64 oracle:
d_k 128 and 256, chunk 64 and 128, d_v 256 (rows normalised in the kernel)
and 512 (per-wave GroupNorm partials and the finishing pass), one segment and
several, an incoming state, a non-zero start position, gammas whose carried
state is rescaled every chunk or never, the flags the schedule takes, an
outgoing state written over the incoming one, and run-to-run determinism.
Tolerance 2e-2 (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu

FUSED = 16  # MSR_FLAG_FUSED

CASES = [  # (B, T, H, dk, dv, chunk); segments per pair in the comment
    (1, 512, 2, 128, 256, 64),     # 8 chunks
    (2, 320, 4, 128, 256, 64),     # 5 chunks
    (1, 2048, 1, 128, 256, 64),    # several segments
    (1, 1024, 2, 256, 256, 64),
    (1, 384, 2, 256, 512, 64),
    (2, 1024, 1, 256, 512, 64),
    (1, 1024, 2, 128, 256, 128),
    (1, 2048, 1, 128, 512, 128),
    (2, 512, 2, 256, 256, 128),
    (1, 2048, 1, 256, 512, 128),
]
# gammas of the fused schedule (a gamma below 0.9 takes the split-score route)
GAMMAS = np.array([0.9, 0.96875, 0.999, 1.0], dtype=np.float32)


def run(q, k, v, g, chunk, s_in=None, flags=0, **kw):
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, flags=flags | FUSED, **kw)
    torch.cuda.synchronize()
    return down(o), down(s)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_fused_vs_oracle(case):
    B, T, H, dk, dv, b = case
    w = mi.Workload("fused", 61, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    for g in (np.resize(mi.gammas(8)[:4], H).astype(np.float32), np.resize(GAMMAS, H).astype(np.float32)):
        note(f"fused {case} gamma {g}: oracle")
        ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=5)
        note(f"fused {case}: gpu")
        o, st = run(q, k, v, g, b, s_in=s, pos0=5)
        eo, es = out_err(o, ro), state_err(st, rs)
        note(f"  O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("flags", [1, 2, 3])  # no rotation / no GroupNorm / neither
@pytest.mark.parametrize("dv", [256, 512])
def test_fused_flags(flags, dv):
    w = mi.Workload("fused-flags", 62, 1, 1024, 2, 128, dv, "bf16", (64,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(2)
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=7, rotate=not (flags & 1), groupnorm=not (flags & 2))
    note(f"fused flags {flags} dv {dv}")
    o, st = run(q, k, v, g, 64, s_in=s, pos0=7, flags=flags)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_fused_large_position():
    """Rotation angles from a start position far past the sequence length
    (the angle reduction is in fp64)."""
    w = mi.Workload("fused-pos", 63, 1, 512, 2, 256, 256, "bf16", (128,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(2)
    pos0 = 3_000_000_017
    th = orc.default_theta(256)  # the same fp32 frequencies on both sides
    ro, rs = orc.recurrent(q, k, v, g, pos0=pos0, theta=th)
    o, st = run(q, k, v, g, 128, pos0=pos0, theta=th)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"fused pos0 {pos0}: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("dv", [256, 512])
def test_fused_state_out_over_state_in_and_determinism(dv):
    """With segments, the outgoing state may overwrite the incoming one (the
    full pass reads a copy the state-only pass set aside); two runs agree
    bit for bit."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.Workload("fused-alias", 64, 1, 4096, 1, 128, dv, "bf16", (64,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(1)
    ro, rs = orc.recurrent(q, k, v, g, s_in=s)
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    outs = []
    for _ in range(2):
        sd = torch.from_numpy(s).to(dev)
        o, st = msr.msr_chunkwise(qd, kd, vd, g, 64, state_in=sd, state_out=sd, flags=FUSED)
        torch.cuda.synchronize()
        outs.append((down(o), down(st)))
    eo, es = out_err(outs[0][0], ro), state_err(outs[0][1], rs)
    note(f"fused alias dv {dv}: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_fused_agrees_with_default_schedule():
    """The two schedules of the same call agree to the tolerance."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.Workload("fused-vs-default", 65, 2, 2048, 4, 256, 512, "bf16", (128,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(4)
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    o1, s1 = msr.msr_chunkwise(qd, kd, vd, g, 128, flags=FUSED)
    o2, s2 = msr.msr_chunkwise(qd, kd, vd, g, 128)
    torch.cuda.synchronize()
    eo, es = out_err(down(o1), down(o2)), state_err(down(s1), down(s2))
    note(f"fused vs default: O {eo:.2e}  state {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
