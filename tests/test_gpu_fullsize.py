"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, checked on sampled (batch, head) pairs that the fp64 oracle
recomputes alone (pairs are independent in every form), plus properties that
hold at any size: the GPU's chunk sizes agree with each other on every pair.

Workloads (seeded, synthetic):
  7B-shaped layer  B=2, T=8192, H=16, d_k=256, d_v=512, bf16, chunk 128 / 256
  decode           B=64, H=16, d_k=256, d_v=512: 2048-token chunkwise prefill
                   (chunk 128) then single-token steps; inputs drawn on the
                   device with torch's seeded generator (2.1e9 values)
  long sequence    B=1, T=131072, H=8, d_k=128, d_v=256, bf16, chunk 64/128/256
Tolerance 2e-2 (bf16 inputs, fp32 accumulation), per-slice max relative error.
"""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, torch_dev, up

pytestmark = pytest.mark.gpu


def slice_err(x, r):
    """max|x - r| / max|r| of one pair's slice."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30))


def oracle_pairs(q, k, v, gamma, pairs, **kw):
    """Oracle recurrence over the sampled pairs only: their slices are stacked
    as the heads of one batch row (each head keeps its own gamma)."""
    sel = lambda x: np.stack([x[b, :, h, :] for b, h in pairs], axis=1)[None]
    g = np.array([gamma[h] for _, h in pairs], dtype=np.float32)
    s_in = kw.pop("s_in", None)
    if s_in is not None:
        s_in = np.stack([s_in[b, h] for b, h in pairs])[None]
    o, s = orc.recurrent(sel(q), sel(k), sel(v), g, s_in=s_in, **kw)
    return {p: (o[0, :, i, :], s[0, i]) for i, p in enumerate(pairs)}


# ---------------------------------------------------------------- 7B shape
PAIRS_7B = [(0, 0), (1, 9), (0, 15), (1, 3), (1, 15)]


@pytest.fixture(scope="module")
def seven_b():
    w = mi.WORKLOADS["7b"]
    note("7B: generating inputs")
    q, k, v = mi.qkv(w)
    g = mi.gammas(w.H)
    note("7B: oracle on sampled pairs", PAIRS_7B)
    ref = oracle_pairs(q, k, v, g, PAIRS_7B)
    return w, q, k, v, g, ref


def run_chunkwise_like_bench(w, q, k, v, g, chunk, flags=0):
    """Same call as the benchmark: preallocated output, state and workspace."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    qd, kd, vd = (up(x, w.dtype, dev) for x in (q, k, v))
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=qd.dtype, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g,
                                        msr.MSR_FORM_CHUNKWISE, chunk, flags=flags), dtype=torch.uint8, device=dev)
    msr.msr_chunkwise(qd, kd, vd, g, chunk, out=o, state_out=s, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return o, s


FUSED = 16  # MSR_FLAG_FUSED: the fused schedule of the chunkwise form


@pytest.mark.parametrize("chunk,flags", [(128, 0), (64, 0), (256, 0), (128, FUSED)])
def test_7b_sampled_pairs_vs_oracle(seven_b, chunk, flags):
    w, q, k, v, g, ref = seven_b
    note(f"7B chunk {chunk} flags {flags}: gpu")
    o, s = run_chunkwise_like_bench(w, q, k, v, g, chunk, flags)
    for (b, h), (ro, rs) in ref.items():
        eo = slice_err(down(o[b, :, h, :]), ro)
        es = slice_err(down(s[b, h]), rs)
        note(f"  pair ({b},{h}): O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_7b_chunk_sizes_agree_on_every_pair(seven_b):
    w, q, k, v, g, _ = seven_b
    torch, _ = torch_dev()
    o1, s1 = run_chunkwise_like_bench(w, q, k, v, g, 128)
    o2, s2 = run_chunkwise_like_bench(w, q, k, v, g, 256)
    # per-pair relative error, computed on the device
    d = (o1.float() - o2.float()).abs().amax(dim=(1, 3))
    r = o2.float().abs().amax(dim=(1, 3))
    eo = float((d / r).max())
    es = float(((s1 - s2).abs().amax(dim=(2, 3)) / s2.abs().amax(dim=(2, 3))).max())
    note(f"7B chunk 128 vs 256 over all pairs: O {eo:.2e}  state {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


# ------------------------------------------------ 7B shape, parallel form
PAIRS_PAR = [(0, 0), (0, 7), (1, 3), (1, 15)]
ROWS_PAR = [0, 1, 127, 128, 129, 4095, 4096, 8191]


def run_parallel_like_bench(w, q, k, v, g, s_in=None):
    """The benchmark's msr_parallel call: preallocated output, state, workspace."""
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    qd, kd, vd = (up(x, w.dtype, dev) for x in (q, k, v))
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=qd.dtype, device=dev)
    s = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    sd = None if s_in is None else torch.from_numpy(s_in).to(dev)
    ws = torch.empty(msr.workspace_size(w.B, w.T, w.H, w.dk, w.dv, msr.MSR_BF16, g,
                                        msr.MSR_FORM_PARALLEL, 0), dtype=torch.uint8, device=dev)
    msr.msr_parallel(qd, kd, vd, g, out=o, state_in=sd, state_out=s, workspace=ws)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("with_state", [False, True])
def test_7b_parallel_sampled_rows_vs_oracle(seven_b, with_state):
    # rows at chunk-like boundaries and at the far end, where gamma^(n-m)
    # underflows fp32 for all but the slowest heads
    w, q, k, v, g, ref = seven_b
    s_in = mi.state(w, 0.05) if with_state else None
    note(f"7B parallel (state in: {with_state}): gpu")
    o, s = run_parallel_like_bench(w, q, k, v, g, s_in)
    for (b, h) in PAIRS_PAR:
        ro = orc.parallel_rows(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], g[h], ROWS_PAR,
                               s_in=None if s_in is None else s_in[b, h])
        eo = slice_err(down(o[b, ROWS_PAR, h, :]), ro)
        note(f"  pair ({b},{h}) rows {ROWS_PAR}: O err {eo:.2e}")
        assert eo < TOL["bf16"]
    # the outgoing state on the pairs the module's oracle ran (zero incoming state)
    if not with_state:
        for (b, h), (_, rs) in ref.items():
            es = slice_err(down(s[b, h]), rs)
            note(f"  pair ({b},{h}): state err {es:.2e}")
            assert es < TOL["bf16"]


def test_7b_parallel_state_in_full_pairs_vs_oracle(seven_b):
    # two whole pairs with an incoming state: gamma^T S_in matters on head 15
    # (gamma^8192 ~ 0.992) and underflows on head 0
    w, q, k, v, g, _ = seven_b
    s_in = mi.state(w, 0.05)
    pairs = [(0, 0), (1, 15)]
    note("7B parallel with state: oracle on", pairs)
    ref = oracle_pairs(q, k, v, g, pairs, s_in=s_in)
    o, s = run_parallel_like_bench(w, q, k, v, g, s_in)
    for (b, h), (ro, rs) in ref.items():
        eo = slice_err(down(o[b, :, h, :]), ro)
        es = slice_err(down(s[b, h]), rs)
        note(f"  pair ({b},{h}): O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_7b_parallel_agrees_with_chunkwise_on_every_pair(seven_b):
    w, q, k, v, g, _ = seven_b
    s_in = mi.state(w, 0.05)
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    o1, s1 = run_parallel_like_bench(w, q, k, v, g, s_in)
    qd, kd, vd = (up(x, w.dtype, dev) for x in (q, k, v))
    o2, s2 = msr.msr_chunkwise(qd, kd, vd, g, 128, state_in=torch.from_numpy(s_in).to(dev))
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs().amax(dim=(1, 3))
    r = o2.float().abs().amax(dim=(1, 3))
    eo = float((d / r).max())
    es = float(((s1 - s2).abs().amax(dim=(2, 3)) / s2.abs().amax(dim=(2, 3))).max())
    note(f"7B parallel vs chunkwise 128 over all pairs: O {eo:.2e}  state {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


# ---------------------------------------------------------------- decode
PAIRS_DEC = [(0, 0), (37, 5), (63, 15)]
DEC_STEPS = 32


def test_decode_full_batch_sampled_pairs_vs_oracle():
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    w = mi.WORKLOADS["decode"]
    g = mi.gammas(w.H)
    note("decode: prefill inputs on the device")
    q = mi.device_normal((w.B, w.T, w.H, w.dk), 3001, dev, torch.bfloat16)
    k = mi.device_normal((w.B, w.T, w.H, w.dk), 3002, dev, torch.bfloat16)
    v = mi.device_normal((w.B, w.T, w.H, w.dv), 3003, dev, torch.bfloat16)
    _, state = msr.msr_chunkwise(q, k, v, g, 128)
    torch.cuda.synchronize()
    host = lambda t, b, h: down(t[b, :, h, :]).astype(np.float32)
    pre = {p: (host(q, *p), host(k, *p), host(v, *p)) for p in PAIRS_DEC}
    del q, k, v
    qs = mi.device_normal((DEC_STEPS, w.B, w.H, w.dk), 3004, dev, torch.bfloat16)
    ks = mi.device_normal((DEC_STEPS, w.B, w.H, w.dk), 3005, dev, torch.bfloat16)
    vs = mi.device_normal((DEC_STEPS, w.B, w.H, w.dv), 3006, dev, torch.bfloat16)
    outs = []
    note(f"decode: {DEC_STEPS} steps, B={w.B}")
    for i in range(DEC_STEPS):
        outs.append(msr.msr_recurrent_step(qs[i], ks[i], vs[i], state, g, w.T + i))
    torch.cuda.synchronize()
    for (b, h) in PAIRS_DEC:
        # the pair's whole sequence (prefill then steps) as one recurrence
        tok = lambda pre_x, xs: np.concatenate([pre_x, down(xs[:, b, h, :]).astype(np.float32)])
        qq = tok(pre[(b, h)][0], qs)[None, :, None]
        kk = tok(pre[(b, h)][1], ks)[None, :, None]
        vv = tok(pre[(b, h)][2], vs)[None, :, None]
        ro, rs = orc.recurrent(qq, kk, vv, g[h:h + 1])
        go = np.stack([down(o[b, h]) for o in outs])
        eo = slice_err(go, ro[0, w.T:, 0, :])
        es = slice_err(down(state[b, h]), rs[0, 0])
        note(f"  pair ({b},{h}): step outputs err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


# ---------------------------------------------------------------- long sequence
PAIRS_LONG = [(0, 0), (0, 7)]


@pytest.fixture(scope="module")
def long_seq():
    w = mi.WORKLOADS["long"]
    note("long: generating inputs")
    q, k, v = mi.qkv(w)
    g = mi.gammas(w.H)
    note("long: oracle on sampled pairs", PAIRS_LONG)
    ref = oracle_pairs(q, k, v, g, PAIRS_LONG)
    return w, q, k, v, g, ref


@pytest.mark.parametrize("chunk,flags", [(64, 0), (128, 0), (256, 0), (64, FUSED), (128, FUSED)])
def test_long_sampled_pairs_vs_oracle(long_seq, chunk, flags):
    w, q, k, v, g, ref = long_seq
    note(f"long chunk {chunk} flags {flags}: gpu")
    o, s = run_chunkwise_like_bench(w, q, k, v, g, chunk, flags)
    for (b, h), (ro, rs) in ref.items():
        eo = slice_err(down(o[b, :, h, :]), ro)
        es = slice_err(down(s[b, h]), rs)
        note(f"  pair ({b},{h}): O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]
