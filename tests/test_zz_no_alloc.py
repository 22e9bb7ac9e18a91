"""msr_chunkwise_noalloc: the chunkwise form with the library's fixed per-GPU
scratch array instead of a caller workspace.  Checked against msr_chunkwise
(same kernels, so the results must agree bit for bit and both must meet the
bf16 tolerance against the fp64 oracle) on two calls in a row, the second
with a smaller input, so the second call runs on scratch the first one left
behind.  Also: a problem whose scratch need exceeds the array is rejected
before anything runs."""
import numpy as np
import pytest

import msr_inputs as mi
from oracle import oracle as orc
from tests.gpu_util import TOL, down, note, out_err, state_err, torch_dev, up

CALLS = [  # (B, T, H, dk, dv, chunk): the second call is smaller than the first
    (2, 1024, 4, 128, 256, 128),
    (1, 256, 2, 64, 128, 64),
]


@pytest.mark.gpu
def test_noalloc_matches_chunkwise_on_two_calls_in_a_row():
    torch, dev = torch_dev()
    import retnet_scale_retention_amd as msr
    for i, (B, T, H, dk, dv, chunk) in enumerate(CALLS):
        w = mi.Workload("noalloc", 90 + i, B, T, H, dk, dv, "bf16", (chunk,))
        q, k, v = mi.qkv(w)
        s_in = mi.state(w, 0.05)
        g = mi.gammas(H)
        need = msr.workspace_size(B, T, H, dk, dv, msr.MSR_BF16, g, msr.MSR_FORM_CHUNKWISE, chunk)
        assert 0 < need <= msr.NOALLOC_SCRATCH_BYTES
        qd, kd, vd = (up(x, "bf16", dev) for x in (q, k, v))
        sd = torch.from_numpy(s_in).to(dev)
        o_ref, s_ref = msr.msr_chunkwise(qd, kd, vd, g, chunk, state_in=sd, pos0=5)
        o = torch.empty_like(o_ref)
        s = torch.empty_like(s_ref)
        note(f"noalloc call {i}: {CALLS[i]}, scratch need {need} bytes")
        msr.msr_chunkwise_noalloc(qd, kd, vd, g, chunk, out=o, state_out=s, state_in=sd, pos0=5)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        ro, rs = orc.chunkwise(q, k, v, g, chunk, s_in=s_in, pos0=5)
        eo, es = out_err(down(o), ro), state_err(down(s), rs)
        note(f"  O err {eo:.2e}  state err {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_noalloc_rejects_a_problem_beyond_the_scratch_array():
    # validation only: nothing is launched and no device is touched
    import ctypes
    import retnet_scale_retention_amd as msr
    from retnet_scale_retention_amd import msr as m
    g = mi.gammas(16)
    d = m._Desc(2, 8192, 16, 256, 512, m.MSR_BF16, g)
    need = msr.workspace_size(2, 8192, 16, 256, 512, m.MSR_BF16, g, m.MSR_FORM_CHUNKWISE, 128)
    assert need > msr.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    s = msr.load().msr_chunkwise_noalloc(d.ref, 128, fake, fake, fake, ctypes.c_void_p(0x20000), None, None, None)
    assert m.STATUS[s] == "MSR_ERR_WORKSPACE"
    assert b"scratch" in msr.load().msr_last_error()
