"""GPU parity of the bf16 MFMA chunkwise kernels against the fp64 oracle,
over every (d_k, chunk) specialisation, one and several value slices, an
incoming state, non-zero start positions and the flags; plus run-to-run
determinism.  Tolerance 2e-2 (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu

CASES = [  # (B, T, H, dk, dv, chunk)
    (2, 192, 2, 64, 64, 64),
    (1, 384, 2, 64, 128, 128),
    (1, 512, 2, 64, 64, 256),
    (1, 256, 2, 128, 64, 64),
    (2, 384, 2, 128, 256, 128),
    (1, 512, 1, 128, 128, 256),
    (1, 192, 2, 256, 64, 64),
    (1, 512, 1, 256, 128, 256),
    (1, 384, 2, 256, 192, 128),
]


def run(q, k, v, g, chunk, s_in=None, **kw):
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, **kw)
    torch.cuda.synchronize()
    return down(o), down(s)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_mfma_chunkwise_vs_oracle(case):
    B, T, H, dk, dv, b = case
    w = mi.Workload("mfma", 31, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(H)
    note(f"mfma case {case}: oracle")
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=3)
    note(f"mfma case {case}: gpu")
    o, st = run(q, k, v, g, b, s_in=s, pos0=3)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("flags", [1, 2])
def test_mfma_flags(flags):
    w = mi.Workload("mfma-flags", 32, 1, 256, 2, 128, 128, "bf16", (128,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(2)
    ro, rs = orc.recurrent(q, k, v, g, rotate=not (flags & 1), groupnorm=not (flags & 2))
    note(f"mfma flags {flags}")
    o, st = run(q, k, v, g, 128, flags=flags)
    assert out_err(o, ro) < TOL["bf16"] and state_err(st, rs) < TOL["bf16"]


def test_mfma_matches_generic_path_and_is_deterministic():
    """The MFMA kernel and the generic kernel (fp32 arithmetic; reached here
    with a chunk of 32, which the MFMA path does not take) agree, and two
    MFMA runs are bitwise identical."""
    w = mi.Workload("mfma-gen", 33, 2, 512, 2, 128, 128, "bf16", (128,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(2)
    note("mfma vs generic")
    o1, s1 = run(q, k, v, g, 128)
    o2, s2 = run(q, k, v, g, 128)
    og, sg = run(q, k, v, g, 32)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    assert out_err(o1, og) < TOL["bf16"] and state_err(s1, sg) < TOL["bf16"]


def test_mfma_state_handoff():
    """chunkwise(T1) -> chunkwise(T2) from the handed-over state equals one
    pass over T1 + T2 (positions continue)."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.Workload("mfma-handoff", 34, 1, 768, 2, 128, 128, "bf16", (128,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(2)
    ro, rs = orc.recurrent(q, k, v, g)
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    o1, s1 = msr.msr_chunkwise(qd[:, :256].contiguous(), kd[:, :256].contiguous(), vd[:, :256].contiguous(), g, 128)
    o2, s2 = msr.msr_chunkwise(qd[:, 256:].contiguous(), kd[:, 256:].contiguous(), vd[:, 256:].contiguous(), g, 128,
                               state_in=s1, pos0=256)
    torch.cuda.synchronize()
    o = np.concatenate([down(o1), down(o2)], 1)
    assert out_err(o, ro) < TOL["bf16"] and state_err(down(s2), rs) < TOL["bf16"]


# Few (pair, slice) workgroups relative to the chunk count: the library splits
# each pair's chunks into segments (a state-only pass for the segment end
# states, then the full pass from the combined incoming states).  Cases run
# with an incoming state and a non-zero start position; the gammas span the
# rescale periods of the carried state (0.75: every 1-2 chunks; 1.0: never).
# (At gamma = 0.5 the bf16 rounding of the rotated q~, k~ alone -- emulated
# on the CPU -- already gives ~2.1e-2: rows whose diagonal score nearly
# cancels have a small spread that GroupNorm amplifies.  The workloads use
# gamma >= 1 - 2^-5, where the same emulation gives ~5e-3.)
SEG_CASES = [  # (B, T, H, dk, dv, chunk)
    (1, 1024, 1, 64, 64, 64),
    (1, 1536, 2, 64, 128, 128),
    (1, 2048, 1, 128, 128, 128),
    (1, 2048, 1, 128, 64, 256),
    (1, 1024, 2, 256, 128, 64),
    (1, 2048, 1, 256, 128, 128),
    (1, 2048, 1, 256, 64, 256),
]
SEG_GAMMAS = np.array([0.75, 0.96875, 0.999, 1.0], dtype=np.float32)


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_mfma_segments_vs_oracle(case):
    B, T, H, dk, dv, b = case
    w = mi.Workload("mfma-seg", 35, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    for gi in range(0, len(SEG_GAMMAS), H):
        g = SEG_GAMMAS[gi:gi + H]
        if len(g) < H:
            g = np.resize(SEG_GAMMAS, H).astype(np.float32)
        note(f"segments {case} gamma {g}: oracle")
        ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=5)
        o, st = run(q, k, v, g, b, s_in=s, pos0=5)
        eo, es = out_err(o, ro), state_err(st, rs)
        note(f"  O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


# The bf16 parallel form (T a multiple of 64) runs its own MFMA kernel: causal
# score blocks per 64-query block with the decay applied in registers, the
# incoming-state term from S_in^T, and the outgoing state as one decayed sum.
PAR_CASES = [  # (B, T, H, dk, dv); d_v a multiple of 256 takes 256-column output slices
    (1, 64, 2, 64, 64),
    (2, 192, 2, 64, 128),
    (1, 512, 2, 128, 64),
    (1, 320, 2, 128, 192),
    (1, 256, 2, 256, 64),
    (1, 512, 1, 256, 128),
    (2, 128, 2, 64, 256),
    (1, 320, 2, 128, 256),
    (1, 192, 2, 256, 512),
]


def run_parallel(q, k, v, g, s_in=None, **kw):
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    o, s = msr.msr_parallel(qd, kd, vd, g, state_in=sd, **kw)
    torch.cuda.synchronize()
    return down(o), down(s)


@pytest.mark.parametrize("case", PAR_CASES, ids=lambda c: "B%dT%dH%ddk%ddv%d" % c)
def test_mfma_parallel_vs_oracle(case):
    B, T, H, dk, dv = case
    w = mi.Workload("mfma-par", 36, B, T, H, dk, dv, "bf16", (T,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(H)
    note(f"parallel {case}: oracle")
    ro, rs = orc.parallel(q, k, v, g, s_in=s, pos0=7)
    o, st = run_parallel(q, k, v, g, s_in=s, pos0=7)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
    # the GPU's parallel and chunkwise forms agree
    oc, sc = run(q, k, v, g, 64, s_in=s, pos0=7)
    assert out_err(o, oc) < TOL["bf16"] and state_err(st, sc) < TOL["bf16"]


@pytest.mark.parametrize("flags", [1, 2])
@pytest.mark.parametrize("dv", [128, 512])
def test_mfma_parallel_flags(flags, dv):
    w = mi.Workload("mfma-par-flags", 37, 1, 256, 2, 128, dv, "bf16", (256,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(2)
    ro, rs = orc.parallel(q, k, v, g, rotate=not (flags & 1), groupnorm=not (flags & 2))
    o, st = run_parallel(q, k, v, g, flags=flags)
    assert out_err(o, ro) < TOL["bf16"] and state_err(st, rs) < TOL["bf16"]


def test_mfma_parallel_state_out_aliases_state_in():
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.Workload("mfma-par-alias", 38, 1, 192, 2, 64, 128, "bf16", (192,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(2)
    ro, rs = orc.parallel(q, k, v, g, s_in=s)
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = torch.from_numpy(s).to(dev)
    o, s2 = msr.msr_parallel(qd, kd, vd, g, state_in=sd, state_out=sd)
    torch.cuda.synchronize()
    assert s2.data_ptr() == sd.data_ptr()
    assert out_err(down(o), ro) < TOL["bf16"] and state_err(down(sd), rs) < TOL["bf16"]


# strong decay: rows dominated by a few tokens, where bf16-rounded q~, k~
# lose the relative accuracy of small scores (the split-scores option)
STRONG = [  # (B, T, H, dk, dv, chunk)
    (2, 256, 2, 64, 128, 64),
    (1, 256, 2, 256, 512, 128),
    (1, 512, 2, 128, 64, 256),
    (1, 512, 1, 256, 128, 256),   # Q~ not staged in LDS by the prep kernel at d_k = b = 256
]


@pytest.mark.parametrize("case", STRONG, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
@pytest.mark.parametrize("gamma", [0.5, 0.25])
def test_mfma_split_scores_strong_decay(case, gamma):
    B, T, H, dk, dv, chunk = case
    import retnet_scale_retention_amd as msr
    w = mi.Workload("strong", 80, B, T, H, dk, dv, "bf16", (chunk,))
    q, k, v = mi.qkv(w)
    g = np.full(H, gamma, np.float32)
    s_in = mi.state(w, 0.5)
    ro, rs = orc.chunkwise(q, k, v, g, chunk, s_in=s_in, pos0=9)
    o1, s1 = run(q, k, v, g, chunk, s_in=s_in, pos0=9)
    o2, s2 = run(q, k, v, g, chunk, s_in=s_in, pos0=9, flags=msr.MSR_FLAG_SPLIT_SCORES)
    e1, e2 = out_err(o1, ro), out_err(o2, ro)
    note(f"gamma={gamma}: O err {e1:.2e} plain, {e2:.2e} split scores; state err {state_err(s2, rs):.2e}")
    assert e2 < TOL["bf16"] and state_err(s2, rs) < TOL["bf16"]
    assert e2 <= e1 * 1.05


@pytest.mark.parametrize("flags", [2, 4, 6])  # no GroupNorm / row-normalised decay / both
def test_mfma_split_scores_with_flags(flags):
    import retnet_scale_retention_amd as msr
    w = mi.Workload("split-flags", 81, 2, 256, 2, 64, 128, "bf16", (64,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(2)
    ro, _ = orc.chunkwise(q, k, v, g, 64, pos0=3, groupnorm=not (flags & 2), rownorm=bool(flags & 4))
    o, _ = run(q, k, v, g, 64, pos0=3, flags=flags | msr.MSR_FLAG_SPLIT_SCORES)
    e = out_err(o, ro)
    note(f"split scores, flags {flags}: O err {e:.2e}")
    assert e < TOL["bf16"]
