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
    # b = 256 with 8 value slices per pair: the full pass prefetches the next
    # chunk's fragment lines into L2 (also with segments)
    (1, 512, 2, 128, 512, 256),
    (1, 2048, 1, 128, 512, 256),
    (1, 512, 1, 256, 512, 256),
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
    # 256-column slices with T a multiple of 256: eight-wave workgroups of 256 queries
    (1, 512, 2, 128, 256),
    (2, 768, 1, 256, 512),
    (1, 256, 3, 64, 256),
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
# lose the relative accuracy of small scores.  Any head below gamma = 0.9
# sends the default call to split scores; these tests call the default.
STRONG_GAMMAS = [0.75, 0.5, 0.25, 0.1]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
@pytest.mark.parametrize("gamma", STRONG_GAMMAS)
def test_mfma_default_call_strong_decay(case, gamma):
    B, T, H, dk, dv, chunk = case
    w = mi.Workload("strong", 80, B, T, H, dk, dv, "bf16", (chunk,))
    q, k, v = mi.qkv(w)
    g = np.full(H, gamma, np.float32)
    s_in = mi.state(w, 0.5)
    ro, rs = orc.chunkwise(q, k, v, g, chunk, s_in=s_in, pos0=9)
    note(f"strong decay {case} gamma={gamma}: gpu")
    o, st = run(q, k, v, g, chunk, s_in=s_in, pos0=9)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_mfma_strong_decay_route_equals_the_flag():
    # the automatic route and the explicit option run the same kernels
    import retnet_scale_retention_amd as msr
    w = mi.Workload("strong-flag", 82, 1, 256, 2, 128, 256, "bf16", (128,))
    q, k, v = mi.qkv(w)
    g = np.array([0.97, 0.4], np.float32)  # one head below the threshold routes the call
    o1, s1 = run(q, k, v, g, 128, pos0=2)
    o2, s2 = run(q, k, v, g, 128, pos0=2, flags=msr.MSR_FLAG_SPLIT_SCORES)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    ro, rs = orc.chunkwise(q, k, v, g, 128, pos0=2)
    assert out_err(o1, ro) < TOL["bf16"] and state_err(s1, rs) < TOL["bf16"]


PAR_STRONG = [  # (B, T, H, dk, dv)
    (2, 192, 2, 64, 128),
    (1, 256, 2, 128, 256),
    (1, 320, 1, 256, 512),
]


@pytest.mark.parametrize("case", PAR_STRONG, ids=lambda c: "B%dT%dH%ddk%ddv%d" % c)
@pytest.mark.parametrize("gamma", STRONG_GAMMAS)
def test_mfma_parallel_default_call_strong_decay(case, gamma):
    B, T, H, dk, dv = case
    w = mi.Workload("par-strong", 83, B, T, H, dk, dv, "bf16", (T,))
    q, k, v = mi.qkv(w)
    g = np.full(H, gamma, np.float32)
    s_in = mi.state(w, 0.5)
    ro, rs = orc.parallel(q, k, v, g, s_in=s_in, pos0=4)
    note(f"parallel strong decay {case} gamma={gamma}: gpu")
    o, st = run_parallel(q, k, v, g, s_in=s_in, pos0=4)
    eo, es = out_err(o, ro), state_err(st, rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


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


ALIAS_SEG = [  # (B, T, H, dk, dv, chunk): 64-column kernels with 4 segments per pair
    (1, 4096, 8, 128, 256, 256),   # chunk_mfma_kernel full pass after its state-only pass
    (1, 2048, 8, 256, 512, 128),   # chunk_ws_kernel full pass after the state-only pass
]


@pytest.mark.parametrize("case", ALIAS_SEG, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_mfma_segmented_state_out_aliases_state_in(case):
    # every segment's workgroup starts from s_in while the last segment's
    # writes s_out: with state_out == state_in the full pass must read only
    # the copy the state-only pass set aside
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    B, T, H, dk, dv, chunk = case
    w = mi.Workload("seg-alias", 84, B, T, H, dk, dv, "bf16", (chunk,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(H)
    note(f"segmented alias {case}: oracle")
    ro, rs = orc.chunkwise(q, k, v, g, chunk, s_in=s)
    qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
    sd = torch.from_numpy(s).to(dev)
    note(f"segmented alias {case}: gpu")
    o, s2 = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, state_out=sd)
    torch.cuda.synchronize()
    assert s2.data_ptr() == sd.data_ptr()
    eo, es = out_err(down(o), ro), state_err(down(sd), rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


# Rows spanning 2 to 8 of the 64-column kernel's slices at b <= 128: the
# slices exchange GroupNorm statistics inside the chunk kernel when its whole
# grid is resident at once.  Cases cover
# an odd slice count, pair counts that are and are not multiples of 8 (the
# workgroups' ticket queues), segments, and b = 64 / 128.  Besides the
# slice-normwise bound, every row must be close on its own, so that one
# mis-normalised row or chunk cannot hide in a slice's norm.
XG_CASES = [  # (B, T, H, dk, dv, chunk)
    (1, 256, 3, 64, 512, 128),
    (2, 512, 4, 64, 320, 64),
    (1, 1024, 2, 256, 448, 128),
    (1, 384, 1, 64, 512, 64),
    (2, 1024, 4, 128, 192, 128),
    # 64 pairs x 8 slices: more workgroups than the GPU holds at once, so the
    # rows take the separate GroupNorm pass instead of the exchange
    (4, 256, 16, 64, 512, 128),
    # b = 64 shapes the wide-slice kernel also takes but would need segments
    # for: they run on this kernel (256 workgroups, no segments)
    (4, 256, 16, 128, 256, 64),
    (2, 256, 16, 256, 512, 64),
]


@pytest.mark.parametrize("case", XG_CASES, ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_mfma_slice_exchange_vs_oracle(case):
    B, T, H, dk, dv, b = case
    w = mi.Workload("mfma-xg", 86, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(H)
    note(f"slice exchange {case}: oracle")
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=7)
    note(f"slice exchange {case}: gpu")
    o1, st = run(q, k, v, g, b, s_in=s, pos0=7)
    o2, _ = run(q, k, v, g, b, s_in=s, pos0=7)
    eo, es = out_err(o1, ro), state_err(st, rs)
    rows = np.linalg.norm((o1 - ro).reshape(-1, dv), axis=1) / np.maximum(np.linalg.norm(ro.reshape(-1, dv), axis=1), 1e-30)
    note(f"  O err {eo:.2e}  state err {es:.2e}  worst row {rows.max():.2e}")
    assert np.array_equal(o1, o2)
    assert eo < TOL["bf16"] and es < TOL["bf16"]
    assert np.isfinite(o1).all() and rows.max() < 0.25


def tick_word(ws, B, T, H, dk, dv, b, k):
    """Counter word k of the exchange (0-7: ticket queues, 8: the call's
    mode, 9: queues whose workgroups have all started, 16 + pair nseg + seg:
    finished workgroups of a call that does not wait), after the MFMA path's
    Q~, K~^T and P^T fragments and slice words in the workspace; for calls
    without segments whose regions are whole multiples of 256 bytes."""
    import torch
    tok = B * T * H
    off = 2 * tok * dk * 2 + tok * b * 2 + tok * (dv // 64) * 8 + 4 * k
    return int(ws[off:off + 4].cpu().view(torch.int32)[0])


@pytest.mark.parametrize("mode", ["off", "no_wait"])
@pytest.mark.parametrize("case", [XG_CASES[0], XG_CASES[1], XG_CASES[4]], ids=lambda c: "B%dT%dH%ddk%ddv%db%d" % c)
def test_mfma_exchange_routes_vs_oracle(case, mode):
    """The two routes that never wait on other workgroups -- a separate
    GroupNorm pass (MSR_EXCHANGE_OFF) and raw rows normalised by the call's
    last workgroup from the exchanged words (MSR_EXCHANGE_NO_WAIT, the route
    of a call that overlaps another) -- against the oracle, and against the
    waiting route to within one more bf16 rounding of the rows."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    B, T, H, dk, dv, b = case
    w = mi.Workload("mfma-xg", 86, B, T, H, dk, dv, "bf16", (b,))
    q, k, v = mi.qkv(w)
    s = mi.state(w, 0.05)
    g = mi.gammas(H)
    note(f"exchange route {mode} {case}: oracle")
    ro, rs = orc.recurrent(q, k, v, g, s_in=s, pos0=7)
    note(f"exchange route {mode} {case}: gpu")
    o_wait, _ = run(q, k, v, g, b, s_in=s, pos0=7)
    ws = torch.empty(msr.workspace_size(B, T, H, dk, dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE, b),
                     dtype=torch.uint8, device=dev)
    msr.set_exchange(msr.MSR_EXCHANGE_OFF if mode == "off" else msr.MSR_EXCHANGE_NO_WAIT)
    try:
        o1, st = run(q, k, v, g, b, s_in=s, pos0=7, workspace=ws)
        o2, _ = run(q, k, v, g, b, s_in=s, pos0=7, workspace=ws)
    finally:
        msr.set_exchange(msr.MSR_EXCHANGE_AUTO)
    eo, es, ew = out_err(o1, ro), state_err(st, rs), out_err(o1, o_wait)
    note(f"  O err {eo:.2e}  state err {es:.2e}  vs waiting route {ew:.2e}")
    if mode == "no_wait" and case == XG_CASES[0]:
        words = [tick_word(ws, *case, i) for i in [8, 9] + list(range(16, 16 + B * H))]
        note(f"  mode, queues started, finished per pair: {words}")
        assert words[:2] == [2, 0] and words[2:] == [dv // 64] * (B * H)
    assert np.array_equal(o1, o2)
    assert eo < TOL["bf16"] and es < TOL["bf16"] and ew < 1e-2
    assert np.isfinite(o1).all()


def test_mfma_slice_exchange_concurrent_calls():
    """Two exchanging calls that overlap on one GPU: call A fills 192 of the
    GPU's workgroup slots for about a millisecond (24 pairs x 8 slices, no
    segments); call B, on a second stream, starts meanwhile on the free CUs.
    A call that finds the exchange claimed (its owner's workgroups not all
    started yet) runs without waiting (mode 2), else it claims it and waits
    (mode 1); both results must hold either way: B against the oracle, A
    against the same call run alone (bitwise when it waited)."""
    import time
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr

    ga = mi.gammas(24)
    A = (1, 32768, 24, 64, 512, 128)
    qa, ka = (mi.device_normal((1, 32768, 24, 64), sd, dev, torch.bfloat16) for sd in (71, 72))
    va = mi.device_normal((1, 32768, 24, 512), 73, dev, torch.bfloat16)
    wsa = torch.empty(msr.workspace_size(*A[:5], msr.MSR_BF16, ga, msr.MSR_FORM_CHUNKWISE, 128), dtype=torch.uint8,
                      device=dev)
    oa_alone = torch.empty_like(va)
    msr.msr_chunkwise(qa, ka, va, ga, 128, out=oa_alone, workspace=wsa, return_state=False)
    torch.cuda.synchronize()

    Bc = (1, 256, 2, 64, 512, 128)
    gb = mi.gammas(2)
    w = mi.Workload("mfma-xg-conc", 87, *Bc[:5], "bf16", (128,))
    q, k, v = mi.qkv(w)
    note("concurrent exchange: oracle")
    ro, _ = orc.recurrent(q, k, v, gb)
    qb, kb, vb = (up(x, "bf16", dev) for x in (q, k, v))
    wsb = torch.empty(msr.workspace_size(*Bc[:5], msr.MSR_BF16, gb, msr.MSR_FORM_CHUNKWISE, 128), dtype=torch.uint8,
                      device=dev)
    ob = torch.empty_like(vb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    note("concurrent exchange: A then B on two streams")
    oa = torch.empty_like(va)
    with torch.cuda.stream(sa):
        msr.msr_chunkwise(qa, ka, va, ga, 128, out=oa, workspace=wsa, return_state=False)
    time.sleep(3e-4)  # A's prologue (~0.1 ms) is over, its chunk kernel runs for ~1 ms
    with torch.cuda.stream(sb):
        msr.msr_chunkwise(qb, kb, vb, gb, 128, out=ob, workspace=wsb, return_state=False)
    torch.cuda.synchronize()
    ma, mb = tick_word(wsa, *A, 8), tick_word(wsb, *Bc, 8)
    e = out_err(down(ob), ro)
    note(f"  modes A {ma} B {mb}; B O err {e:.2e}")
    assert ma in (1, 2) and mb in (1, 2)
    if ma == 1:
        assert torch.equal(oa, oa_alone)
    else:
        assert out_err(down(oa), down(oa_alone)) < 1e-2
    assert np.isfinite(down(ob)).all() and e < TOL["bf16"]
