"""Error statuses of the C ABI that the host decides before any GPU work (no GPU needed): bad model
descriptions, NULL pointers, out-of-range options and plan arguments. The statuses that need an
engine (MK_ERR_NO_SCHEDULE, MK_ERR_SCHEDULE_STALE, MK_ERR_INVALID_ARG from mk_decode_step) are in
test_gpu_abi_errors.py."""

import ctypes

import pytest

from decode_megakernel_03_amd import mk, synth


def _desc(**over):
    wl = synth.workload("tiny")
    d = mk.model_desc(wl, num_pages=16, max_pages_per_seq=8, max_batch=1)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _create(desc, ptrs=None):
    h = ctypes.c_void_p()
    ptrs = ptrs if ptrs is not None else mk.WeightPtrs()
    return mk.LIB.mk_create(ctypes.byref(desc) if desc is not None else None, ctypes.byref(ptrs), ctypes.byref(h)), h


@pytest.mark.parametrize("over,status", [
    (dict(abi_version=99), mk.MK_ERR_INVALID_ARG),
    (dict(n_layers=0), mk.MK_ERR_INVALID_ARG),
    (dict(max_batch=9), mk.MK_ERR_INVALID_ARG),
    (dict(max_batch=0), mk.MK_ERR_INVALID_ARG),
    (dict(page_size=32), mk.MK_ERR_UNSUPPORTED),
    (dict(hidden=512), mk.MK_ERR_UNSUPPORTED),
    (dict(rms_eps=0.0), mk.MK_ERR_INVALID_ARG),
    (dict(rope_theta=-1.0), mk.MK_ERR_INVALID_ARG),
])
def test_create_rejects_bad_descriptions(over, status):
    st, h = _create(_desc(**over))
    assert st == status and not h.value


def test_create_rejects_null_arguments():
    st, h = _create(None)
    assert st == mk.MK_ERR_INVALID_ARG and not h.value
    st, h = _create(_desc())                     # every weight pointer NULL
    assert st == mk.MK_ERR_INVALID_ARG and not h.value
    assert mk.LIB.mk_create(ctypes.byref(_desc()), ctypes.byref(mk.WeightPtrs()), None) == mk.MK_ERR_INVALID_ARG


def test_engine_calls_reject_a_null_engine():
    assert mk.LIB.mk_set_options(None, ctypes.byref(mk.Options())) == mk.MK_ERR_INVALID_ARG
    arr = (ctypes.c_int32 * 1)(65)
    assert mk.LIB.mk_build_schedule(None, 1, arr) == mk.MK_ERR_INVALID_ARG
    assert mk.LIB.mk_decode_step(None, None, None, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert mk.LIB.mk_set_step_outputs(None, None, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert mk.LIB.mk_sync(None) == mk.MK_ERR_INVALID_ARG
    assert mk.LIB.mk_reset(None) == mk.MK_ERR_INVALID_ARG
    buf = ctypes.create_string_buffer(64)
    assert mk.LIB.mk_get_error(None, buf, 64) == mk.MK_ERR_INVALID_ARG and buf.value == b"NULL engine"
    mk.LIB.mk_destroy(None)                      # a no-op


def test_plan_build_rejects_bad_arguments():
    d = _desc()
    h = ctypes.c_void_p()
    lens = (ctypes.c_int32 * 2)(65, 65)
    P32 = ctypes.POINTER(ctypes.c_int32)
    ok = ctypes.cast(lens, P32)
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 2, ok, 64, 0, 0, 1, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG  # batch > max_batch
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 1, ok, 0, 0, 0, 1, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG   # no workers
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 1, None, 64, 0, 0, 1, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG
    too_long = (ctypes.c_int32 * 1)(8 * 16 + 1)                                                           # > max_pages * 16
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 1, ctypes.cast(too_long, P32), 64, 0, 0, 1, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG
    zero = (ctypes.c_int32 * 1)(0)
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 1, ctypes.cast(zero, P32), 64, 0, 0, 1, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG
    one = ctypes.cast((ctypes.c_int32 * 1)(65), P32)
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 1, one, 64, 0, 0, 0, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG   # rows_per_seq 0
    assert mk.LIB.mk_plan_build(ctypes.byref(d), 1, one, 64, 0, 0, 2, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG   # > batch
    assert not h.value


def test_engine_finalizer_makes_no_library_call_when_closed_or_at_shutdown(monkeypatch):
    """Engine.__del__ must not call into the library for a closed engine or while the interpreter
    shuts down (the runtime may be gone), and must work after the module's globals were cleared."""
    calls = []
    monkeypatch.setattr(mk.Engine, "close", lambda self: calls.append(self.h))
    e = mk.Engine.__new__(mk.Engine)
    e.h = None
    monkeypatch.setattr(mk, "_finalizing", None)      # module teardown clears globals
    e.__del__()
    e.h = 7
    e.__del__(_finalizing=lambda: True)
    assert calls == []
    e.__del__(_finalizing=lambda: False)
    assert calls == [7]
    e.h = None
