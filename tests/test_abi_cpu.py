"""CPU-only checks of the C ABI: the library loads, exports what
include/msr.h declares, and rejects invalid calls before touching a GPU."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import retnet_scale_retention_amd as msr
from retnet_scale_retention_amd import msr as m

ROOT = Path(__file__).resolve().parents[1]
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation


def header_functions():
    text = (ROOT / "include" / "msr.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = msr.load()
    names = header_functions()
    assert set(names) == set(m.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.msr_abi_version() == 6


def test_problem_struct_layout_matches_the_header():
    # the binding's struct mirrors msr_problem field by field (pos_rows last)
    names = [f[0] for f in m.Problem._fields_]
    assert names == ["B", "T", "H", "dk", "dv", "dtype", "gamma", "theta", "scale", "gn_eps", "pos0", "flags",
                     "pos_rows"]
    assert m.Problem.pos_rows.offset == 64 and ctypes.sizeof(m.Problem) == 72


def desc(**kw):
    base = dict(B=2, T=64, H=4, dk=16, dv=32, dtype=m.MSR_BF16, gamma=np.full(4, 0.9))
    base.update(kw)
    return m._Desc(**base)


def status_ws(d, form=m.MSR_FORM_CHUNKWISE, chunk=16):
    n = ctypes.c_size_t(12345)
    s = msr.load().msr_workspace_size(d.ref, form, chunk, ctypes.byref(n))
    return s, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(dk=15), m.STATUS.get(-2)), (dict(dk=0), "MSR_ERR_SHAPE"), (dict(dk=1024), "MSR_ERR_SHAPE"),
    (dict(dv=6), "MSR_ERR_SHAPE"), (dict(dv=2048), "MSR_ERR_SHAPE"), (dict(H=0, gamma=np.zeros(0)), "MSR_ERR_SHAPE"),
    (dict(B=-1), "MSR_ERR_SHAPE"), (dict(dtype=7), "MSR_ERR_DTYPE"),
    (dict(gamma=np.array([0.9, 0.9, 0.9, 1.5])), "MSR_ERR_INVALID_ARG"),
    (dict(gamma=np.array([0.9, 0.0, 0.9, 0.9])), "MSR_ERR_INVALID_ARG"),
    (dict(gamma=np.array([0.9, np.nan, 0.9, 0.9])), "MSR_ERR_INVALID_ARG"),
    (dict(eps=-1.0), "MSR_ERR_INVALID_ARG"), (dict(pos0=-3), "MSR_ERR_INVALID_ARG"),
    (dict(flags=32), "MSR_ERR_INVALID_ARG"), (dict(scale=float("inf")), "MSR_ERR_INVALID_ARG"),
])
def test_invalid_problems_are_rejected(kw, code):
    s, n = status_ws(desc(**kw))
    assert m.STATUS[s] == code
    assert n == 12345  # untouched on error
    assert msr.load().msr_last_error().decode()


def test_workspace_bytes_matches_workspace_size():
    lib = msr.load()
    for form, chunk in ((m.MSR_FORM_CHUNKWISE, 16), (m.MSR_FORM_PARALLEL, 0), (m.MSR_FORM_STEP, 0),
                        (m.MSR_FORM_BACKWARD, 16), (m.MSR_FORM_QKV_CHUNKWISE, 16)):
        d = desc(T=1) if form == m.MSR_FORM_STEP else desc()
        s, n = status_ws(d, form, chunk)
        assert s == 0
        assert lib.msr_workspace_bytes(d.ref, form, chunk) == n
    # an invalid problem gives 0 and leaves the reason behind
    assert lib.msr_workspace_bytes(desc(dk=15).ref, m.MSR_FORM_CHUNKWISE, 16) == 0
    assert b"dk" in lib.msr_last_error()


@pytest.mark.parametrize("form,chunk", [(m.MSR_FORM_CHUNKWISE, 64), (m.MSR_FORM_PARALLEL, 0)])
def test_strong_decay_workspace_covers_the_split_route(form, chunk):
    # any head with gamma < 0.9 routes a bf16 matrix-core call to split scores,
    # whose workspace adds Q~ and K~ as hi and lo bf16 parts (4 x B T H dk x 2 bytes)
    kw = dict(B=1, T=256, H=2, dk=64, dv=64)
    _, weak = status_ws(desc(**kw, gamma=np.array([0.97, 0.9])), form, chunk)
    _, strong = status_ws(desc(**kw, gamma=np.array([0.97, 0.5])), form, chunk)
    assert strong > weak and strong >= 4 * 256 * 2 * 64 * 2
    _, flag = status_ws(desc(**kw, gamma=np.array([0.97, 0.9]), flags=m.MSR_FLAG_SPLIT_SCORES), m.MSR_FORM_CHUNKWISE, 64)
    if form == m.MSR_FORM_CHUNKWISE:
        assert strong == flag


def test_chunk_need_not_divide_T():
    # a last chunk shorter than b takes the remaining tokens
    d = desc(T=96)
    assert status_ws(d, chunk=32)[0] == 0
    s40, n40 = status_ws(d, chunk=40)
    s32, n32 = status_ws(d, chunk=32)
    assert s40 == 0 and n40 > 0
    assert m.STATUS[status_ws(d, chunk=0)[0]] == "MSR_ERR_SHAPE"


def test_misaligned_row_positions_are_rejected():
    d = desc()
    d.p.pos_rows = 0x10004  # 4-byte aligned only; never dereferenced
    assert m.STATUS[status_ws(d)[0]] == "MSR_ERR_INVALID_ARG"
    assert "pos_rows" in msr.load().msr_last_error().decode()


def test_workspace_sizes_are_stable_and_step_needs_none():
    d = desc()
    s1, n1 = status_ws(d, m.MSR_FORM_CHUNKWISE, 16)
    s2, n2 = status_ws(d, m.MSR_FORM_PARALLEL, 0)
    assert s1 == 0 and s2 == 0 and n1 > 0 and n2 > 0
    s3, n3 = status_ws(desc(T=1), m.MSR_FORM_STEP, 0)
    assert s3 == 0 and n3 == 0
    assert m.STATUS[status_ws(desc(T=4), m.MSR_FORM_STEP, 0)[0]] == "MSR_ERR_SHAPE"


def test_calls_validate_pointers_before_any_launch():
    lib = msr.load()
    d = desc()
    null = ctypes.c_void_p()
    # missing tensors
    s = lib.msr_parallel(d.ref, null, FAKE, FAKE, FAKE, null, null, FAKE, 1 << 40, null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG"
    # misaligned tensor
    s = lib.msr_chunkwise(d.ref, 16, ctypes.c_void_p(0x10002), FAKE, FAKE, ctypes.c_void_p(0x20000),
                          null, null, FAKE, 1 << 40, null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG"
    # O aliasing Q
    s = lib.msr_chunkwise(d.ref, 16, FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), FAKE,
                          null, null, FAKE, 1 << 40, null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG"
    # workspace too small / missing
    O = ctypes.c_void_p(0x40000)
    s = lib.msr_chunkwise(d.ref, 16, FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), O,
                          null, null, FAKE, 16, null)
    assert m.STATUS[s] == "MSR_ERR_WORKSPACE"
    s = lib.msr_parallel(d.ref, FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), O,
                         null, null, null, 0, null)
    assert m.STATUS[s] == "MSR_ERR_WORKSPACE"
    # decode step: T must be 1, o must not alias the state
    s = lib.msr_recurrent_step(desc(T=2).ref, FAKE, FAKE, FAKE, O, FAKE, null)
    assert m.STATUS[s] == "MSR_ERR_SHAPE"
    s = lib.msr_recurrent_step(desc(T=1).ref, FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000),
                               O, O, null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG"
    assert "alias" in lib.msr_last_error().decode()


def test_qkv_calls_validate_before_any_launch():
    lib = msr.load()
    null = ctypes.c_void_p()
    outs = [ctypes.c_void_p(0x50000 + 0x10000 * i) for i in range(3)]
    # fp32 is not taken
    s = lib.msr_qkv_projection(desc(dtype=m.MSR_F32).ref, 64, FAKE, FAKE, FAKE, FAKE, *outs, null)
    assert m.STATUS[s] == "MSR_ERR_UNSUPPORTED"
    # d_model must be a positive multiple of 64
    for dm in (0, 48, 100):
        s = lib.msr_qkv_projection(desc().ref, dm, FAKE, FAKE, FAKE, FAKE, *outs, null)
        assert m.STATUS[s] == "MSR_ERR_SHAPE"
    # missing or misaligned input, output aliasing an input
    s = lib.msr_qkv_projection(desc().ref, 64, null, FAKE, FAKE, FAKE, *outs, null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG"
    s = lib.msr_qkv_projection(desc().ref, 64, ctypes.c_void_p(0x10008), FAKE, FAKE, FAKE, *outs, null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG"
    s = lib.msr_qkv_projection(desc().ref, 64, FAKE, FAKE, FAKE, FAKE, FAKE, outs[1], outs[2], null)
    assert m.STATUS[s] == "MSR_ERR_INVALID_ARG" and "alias" in lib.msr_last_error().decode()
    # the composite needs its workspace: Q~, K~, V plus the chunkwise form's
    s, n = status_ws(desc(), m.MSR_FORM_QKV_CHUNKWISE, 16)
    s1, n1 = status_ws(desc(), m.MSR_FORM_CHUNKWISE, 16)
    assert s == 0 and s1 == 0 and n >= n1 + 2 * 64 * 4 * (2 * 16 + 32)
    s = lib.msr_qkv_chunkwise(desc().ref, 16, 64, FAKE, FAKE, FAKE, FAKE, outs[0], null, null, FAKE, 16, null)
    assert m.STATUS[s] == "MSR_ERR_WORKSPACE"


def test_empty_problems_need_no_workspace_and_launch_nothing():
    lib = msr.load()
    null = ctypes.c_void_p()
    d = desc(B=0)
    s = lib.msr_qkv_chunkwise(d.ref, 16, 64, null, null, null, null, null, null, null, null, 0, null)
    assert m.STATUS[s] == "MSR_OK", lib.msr_last_error().decode()
    s = lib.msr_qkv_projection(d.ref, 64, null, null, null, null, null, null, null, null)
    assert m.STATUS[s] == "MSR_OK"
    s = lib.msr_chunkwise(d.ref, 16, null, null, null, null, null, null, null, 0, null)
    assert m.STATUS[s] == "MSR_OK"


def test_null_problem_and_bytes():
    lib = msr.load()
    n = ctypes.c_size_t(0)
    assert m.STATUS[lib.msr_workspace_size(None, 1, 16, ctypes.byref(n))] == "MSR_ERR_INVALID_ARG"
    assert m.STATUS[lib.msr_workspace_size(desc().ref, 1, 16, None)] == "MSR_ERR_INVALID_ARG"
    assert m.STATUS[lib.msr_workspace_size(desc().ref, 9, 16, ctypes.byref(n))] == "MSR_ERR_INVALID_ARG"


def test_exchange_mode_accepts_its_three_values_only():
    lib = msr.load()
    for bad in (-1, 3, 1 << 20):
        assert m.STATUS[lib.msr_set_exchange(bad)] == "MSR_ERR_INVALID_ARG"
        assert "exchange mode" in lib.msr_last_error().decode()
    for mode in (m.MSR_EXCHANGE_OFF, m.MSR_EXCHANGE_NO_WAIT, m.MSR_EXCHANGE_AUTO):
        msr.set_exchange(mode)
    with pytest.raises(m.MsrError):
        msr.set_exchange(7)
