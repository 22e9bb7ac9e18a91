"""GPU parity of the batched-serving features: per-batch-row start
positions (pos_rows), a last chunk shorter than b (b not dividing T), and
multi-token decode steps carried through the state.  Each batch row is an
independent sequence, so the reference is the fp64 oracle's plain parallel
definition run on that row alone, at that row's start position.
Tolerance as in the other parity tests: 1e-4 (fp32), 2e-2 (bf16)."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

pytestmark = pytest.mark.gpu


def _msr():
    import retnet_scale_retention_amd as msr
    return msr


def oracle_rows(q, k, v, g, pos, s_in=None):
    """The oracle's parallel form, batch row b at start position pos[b]."""
    outs, states = [], []
    for b in range(q.shape[0]):
        sb = None if s_in is None else s_in[b:b + 1]
        o, s = orc.parallel(q[b:b + 1], k[b:b + 1], v[b:b + 1], g, pos0=int(pos[b]), s_in=sb)
        outs.append(o)
        states.append(s)
    return np.concatenate(outs), np.concatenate(states)


# (name, B, T, H, dk, dv, dtype, chunk): MFMA-path shapes and general-path shapes
ROW_CASES = [
    ("bf16-mfma-b64", 3, 256, 2, 64, 128, "bf16", 64),
    ("bf16-mfma-b128", 2, 256, 2, 128, 64, "bf16", 128),
    ("f32-general", 3, 48, 2, 16, 16, "f32", 16),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=[c[0] for c in ROW_CASES])
@pytest.mark.parametrize("form", ["chunkwise", "parallel"])
def test_row_positions_vs_oracle(case, form):
    name, B, T, H, dk, dv, dtype, chunk = case
    torch, dev = torch_dev()
    msr = _msr()
    w = mi.Workload("rows-" + name, 40, B, T, H, dk, dv, dtype, (chunk,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s_in = mi.state(w, 0.5)
    pos = np.array([0, 1000, 37][:B], dtype=np.int64)
    ro, rs = oracle_rows(q, k, v, g, pos, s_in)
    qd, kd, vd = (up(x, dtype, dev) for x in (q, k, v))
    sd = torch.from_numpy(s_in).to(dev)
    pd = torch.from_numpy(pos).to(dev)
    note(f"{name} {form}: positions {pos.tolist()}")
    if form == "chunkwise":
        o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, pos_rows=pd)
    else:
        o, s = msr.msr_parallel(qd, kd, vd, g, state_in=sd, pos_rows=pd)
    torch.cuda.synchronize()
    eo, es = out_err(down(o), ro), state_err(down(s), rs)
    note(f"  O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
    # the same call with pos_rows = pos0 everywhere equals the pos0 call
    o2, _ = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, pos0=37,
                              pos_rows=torch.full((B,), 37, dtype=torch.int64, device=dev))
    o3, _ = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, pos0=37)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3)


# (name, B, T, H, dk, dv, dtype, chunk) with chunk not dividing T
PARTIAL_CASES = [
    ("bf16-T200-b64", 2, 200, 2, 64, 128, "bf16", 64),
    ("bf16-T100-b128", 1, 100, 2, 128, 64, "bf16", 128),  # one chunk, shorter than b
    ("f32-T50-b16", 1, 50, 2, 16, 16, "f32", 16),
    ("f32-T7-b3", 2, 7, 1, 8, 8, "f32", 3),
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=[c[0] for c in PARTIAL_CASES])
def test_partial_last_chunk_vs_oracle(case):
    name, B, T, H, dk, dv, dtype, chunk = case
    torch, dev = torch_dev()
    msr = _msr()
    w = mi.Workload("partial-" + name, 41, B, T, H, dk, dv, dtype, (chunk,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s_in = mi.state(w, 0.5)
    ro, rs = orc.parallel(q, k, v, g, s_in=s_in, pos0=5)
    qd, kd, vd = (up(x, dtype, dev) for x in (q, k, v))
    o, s = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=torch.from_numpy(s_in).to(dev), pos0=5)
    torch.cuda.synchronize()
    eo, es = out_err(down(o), ro), state_err(down(s), rs)
    note(f"{name}: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


def test_ragged_decode_steps_vs_oracle():
    """Single-token steps for sequences at different positions (one position
    per batch row), state carried in place."""
    torch, dev = torch_dev()
    msr = _msr()
    B, H, dk, dv, steps = 4, 2, 64, 128, 6
    w = mi.Workload("ragged-decode", 42, B, steps, H, dk, dv, "bf16", (1,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s_in = mi.state(w, 0.5)
    pos = np.array([0, 17, 2048, 5], dtype=np.int64)
    ro, rs = oracle_rows(q, k, v, g, pos, s_in)
    st = torch.from_numpy(s_in).to(dev)
    outs = []
    for t in range(steps):
        pd = torch.from_numpy(pos + t).to(dev)
        o = msr.msr_recurrent_step(up(q[:, t], "bf16", dev).contiguous(), up(k[:, t], "bf16", dev).contiguous(),
                                   up(v[:, t], "bf16", dev).contiguous(), st, g, pd)
        outs.append(down(o))
    torch.cuda.synchronize()
    eo, es = out_err(np.stack(outs, 1), ro), state_err(down(st), rs)
    note(f"ragged decode: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("tokens_per_step", [1, 4, 16])
def test_multi_token_steps_vs_oracle(tokens_per_step):
    """Serving loop: each step feeds the next tokens_per_step tokens of every
    sequence (rows at different positions) through msr_chunkwise with the
    state carried; the outputs equal the oracle's single pass per row."""
    torch, dev = torch_dev()
    msr = _msr()
    B, T, H, dk, dv = 3, 48, 2, 64, 128
    w = mi.Workload("multi-step", 43, B, T, H, dk, dv, "bf16", (tokens_per_step,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    pos = np.array([3, 300, 0], dtype=np.int64)
    ro, rs = oracle_rows(q, k, v, g, pos)
    st = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=dev)
    outs = []
    for t0 in range(0, T, tokens_per_step):
        sl = slice(t0, t0 + tokens_per_step)
        qd, kd, vd = (up(np.ascontiguousarray(x[:, sl]), "bf16", dev) for x in (q, k, v))
        pd = torch.from_numpy(pos + t0).to(dev)
        o, _ = msr.msr_chunkwise(qd, kd, vd, g, tokens_per_step, state_in=st, state_out=st, pos_rows=pd)
        outs.append(down(o))
    torch.cuda.synchronize()
    eo, es = out_err(np.concatenate(outs, 1), ro), state_err(down(st), rs)
    note(f"{tokens_per_step} tokens per step: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("T", [2, 9, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("form", ["chunkwise", "parallel"])
@pytest.mark.parametrize("with_state", [False, True])
def test_short_calls_vs_oracle(T, dtype, form, with_state):
    """Calls of at most 16 tokens run the recurrence in one pass over the
    state (any b); separate state_in and state_out buffers."""
    torch, dev = torch_dev()
    msr = _msr()
    B, H, dk, dv = 2, 3, 32, 64
    w = mi.Workload(f"short-{T}-{dtype}", 44, B, T, H, dk, dv, dtype, (T,))
    q, k, v = mi.qkv(w)
    g = mi.gammas(H)
    s_in = mi.state(w, 0.5) if with_state else None
    ro, rs = orc.parallel(q, k, v, g, s_in=s_in, pos0=11)
    qd, kd, vd = (up(x, dtype, dev) for x in (q, k, v))
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    if form == "chunkwise":
        o, s = msr.msr_chunkwise(qd, kd, vd, g, 3, state_in=sd, pos0=11)
    else:
        o, s = msr.msr_parallel(qd, kd, vd, g, state_in=sd, pos0=11)
    torch.cuda.synchronize()
    eo, es = out_err(down(o), ro), state_err(down(s), rs)
    note(f"T={T} {dtype} {form} state={with_state}: O err {eo:.2e}  state err {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
    if sd is not None:  # the incoming state is left untouched
        assert np.array_equal(down(sd), s_in.astype(np.float64))


def test_decode_steps_captured_in_a_hip_graph_match_eager():
    # the benchmark's decode loop runs as one captured HIP graph; every replay
    # (with eager work and synchronisations between replays) must reproduce
    # the eagerly launched steps bit for bit
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    B, H, dk, dv, n = 4, 2, 128, 256, 6
    w = mi.Workload("graph-decode", 95, B, 1, H, dk, dv, "bf16", (1,))
    g = mi.gammas(H)
    s0 = torch.from_numpy(mi.state(w, 0.1)).to(dev)
    qs = mi.device_normal((n, B, H, dk), 9501, dev, torch.bfloat16)
    ks = mi.device_normal((n, B, H, dk), 9502, dev, torch.bfloat16)
    vs = mi.device_normal((n, B, H, dv), 9503, dev, torch.bfloat16)
    st_e = s0.clone()
    outs_e = [msr.msr_recurrent_step(qs[i], ks[i], vs[i], st_e, g, 10 + i) for i in range(n)]
    st_g = s0.clone()
    outs_g = [torch.empty_like(outs_e[0]) for _ in range(n)]
    torch.cuda.synchronize()
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        for i in range(n):
            msr.msr_recurrent_step(qs[i], ks[i], vs[i], st_g, g, 10 + i, out=outs_g[i])
    for rep in range(3):
        st_g.copy_(s0)
        for t in outs_g:
            t.zero_()
        torch.cuda.synchronize()
        gph.replay()
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        for i in range(n):
            assert torch.equal(outs_g[i], outs_e[i]), (rep, i)
        assert torch.equal(st_g, st_e), rep
