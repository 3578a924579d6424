"""Host-side statuses of mk_decode_step through the C ABI on a real engine: MK_ERR_NO_SCHEDULE,
MK_ERR_INVALID_ARG and MK_ERR_SCHEDULE_STALE are returned before anything is launched, and leave the
engine usable; the binding's Engine rebuilds a stale schedule and decoding goes on (checked against
the oracle after the rebuild)."""

import copy
import sys

import numpy as np
import pytest
import torch

from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _engine(extra_steps, max_pages=None):
    from decode_megakernel_03_amd import mk
    wl = synth.workload("tiny")
    s = harness.tiny_setup(wl)
    bt, num_pages = synth.make_block_tables(s["ctx"], extra_steps, wl.page_size)
    s["block_tables"], s["num_pages"] = bt, num_pages
    s["k"], s["v"] = synth.make_kv(wl, num_pages)
    wd = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in s["w"].items() if k != "layers"}
    wd["layers"] = [{k: (v.cuda() if torch.is_tensor(v) else v) for k, v in lw.items()} for lw in s["w"]["layers"]]
    kd = [t.cuda() for t in s["k"]]
    vd = [t.cuda() for t in s["v"]]
    eng = mk.Engine(wl, wd, kd, vd, num_pages, max_pages or bt.shape[1], max_batch=1)
    return wl, s, eng, kd, vd


def _inputs(s, step):
    pos = s["ctx"].astype(np.int64) + step
    return (torch.from_numpy(s["tokens"].astype(np.int32)).cuda(), torch.from_numpy(pos.astype(np.int32)).cuda(),
            torch.from_numpy(s["block_tables"]).cuda(), torch.from_numpy((pos + 1).astype(np.int32)).cuda())


def test_no_schedule_and_null_inputs():
    from decode_megakernel_03_amd import mk
    say("test_no_schedule_and_null_inputs: tiny engine, no kernel launched")
    wl, s, eng, _, _ = _engine(4)
    tok, pos, bt, lens = _inputs(s, 0)
    logits = torch.zeros(1, wl.vocab, dtype=torch.float32, device="cuda")
    assert mk.mk_decode_step(eng.h, tok, pos, bt, lens, logits) == mk.MK_ERR_NO_SCHEDULE
    st, msg = mk.mk_get_error(eng.h)
    assert st == mk.MK_OK and "no schedule" in msg
    eng.build_schedule((s["ctx"] + 1).tolist())
    assert mk.mk_decode_step(eng.h, None, pos, bt, lens, logits) == mk.MK_ERR_INVALID_ARG
    assert mk.mk_decode_step(eng.h, tok, pos, bt, lens, None) == mk.MK_ERR_INVALID_ARG     # the model has an lm_head
    import ctypes
    assert mk.LIB.mk_build_schedule(eng.h, 2, (ctypes.c_int32 * 2)(65, 65)) == mk.MK_ERR_INVALID_ARG   # > max_batch
    with pytest.raises(mk.MkError):
        mk.mk_set_options(eng.h, workers_per_cu=9)
    # none of that launched anything or broke the engine: one real step runs and matches the oracle
    eng.set_step_outputs()
    assert mk.mk_decode_step(eng.h, tok, pos, bt, lens, logits) == mk.MK_OK
    eng.sync()
    import oracle
    ref = oracle.decode_step(harness.dims_of(wl), harness.dense_weights(s["w"]), harness.host_kv(s["k"], s["v"]),
                             s["tokens"], s["ctx"].copy(), s["block_tables"], s["ctx"] + 1)
    assert np.abs(logits.cpu().numpy() - ref.logits).max() <= 2e-2
    eng.close()


def test_schedule_stale_is_refused_before_launch():
    """max_pages_per_seq 5 (80 positions): context 64 leaves room for exactly 16 steps; the 17th is
    refused on the host with MK_ERR_SCHEDULE_STALE, and a rebuild beyond the pages is refused too."""
    from decode_megakernel_03_amd import mk
    say("test_schedule_stale_is_refused_before_launch: tiny engine, 16 valid steps then a refusal")
    wl, s, eng, _, _ = _engine(16, max_pages=5)
    eng.build_schedule((s["ctx"] + 1).tolist())
    assert eng.plan_info().key_capacity_min == 80
    logits = torch.zeros(1, wl.vocab, dtype=torch.float32, device="cuda")
    for step in range(16):
        assert mk.mk_decode_step(eng.h, *_inputs(s, step), logits) == mk.MK_OK
    eng.sync()
    assert mk.mk_decode_step(eng.h, *_inputs(s, 16), logits) == mk.MK_ERR_SCHEDULE_STALE
    st, msg = mk.mk_get_error(eng.h)
    assert st == mk.MK_OK and "capacity 80" in msg
    with pytest.raises(mk.MkError):
        eng.build_schedule([81])                 # longer than the block table allows
    eng.close()


def _run_long(refresh_off):
    """1100 greedy steps of the small model from context 64 through Engine.step, with the oracle
    (teacher-forced on the GPU's tokens and KV cache) at the first rebuild and at the last step."""
    from decode_megakernel_03_amd import mk
    import oracle
    n_steps = 1100
    wl, s, eng, kd, vd = _engine(n_steps + 1)
    eng.build_schedule((s["ctx"] + 1).tolist())
    cap = eng.plan_info().key_capacity_min
    refresh = eng.refresh_keys
    assert refresh == eng.plan_info().split_keys // 4 and refresh > 0
    if refresh_off:
        eng.refresh_keys = 1 << 30                                    # (for the first schedule only)
        assert cap - int(s["ctx"][0]) - 1 < n_steps                   # a rebuild is needed
        first = cap - int(s["ctx"][0])                                # first step refused by the old schedule
        expect = 1 + (n_steps - 1 - first) // refresh                 # (the new schedule refreshes again)
    else:
        first = refresh                                               # the step that rebuilds first
        expect = (n_steps - 1) // refresh
    argmax = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng.set_step_outputs(argmax_out=argmax)
    logits = torch.zeros(1, wl.vocab, dtype=torch.float32, device="cuda")
    dims = harness.dims_of(wl)
    dw = harness.dense_weights(s["w"])
    bt = torch.from_numpy(s["block_tables"]).cuda()
    tok = s["tokens"].astype(np.int64)
    for step in range(n_steps):
        check = step in (first, n_steps - 1)
        kv0 = harness.host_kv(kd, vd) if check else None
        pos = s["ctx"].astype(np.int64) + step
        eng.step(torch.from_numpy(tok.astype(np.int32)).cuda(), torch.from_numpy(pos.astype(np.int32)).cuda(), bt,
                 torch.from_numpy((pos + 1).astype(np.int32)).cuda(), logits)
        if check:
            eng.sync()
            ref = oracle.decode_step(dims, dw, copy.deepcopy(kv0), tok, pos, s["block_tables"], pos + 1)
            d = np.abs(logits.cpu().numpy() - ref.logits).max()
            say(f"  step {step} (position {int(pos[0])}): max|dlogit| {d:.2e}, rebuilds so far {eng.rebuilds}")
            assert d <= 2e-2
            assert int(argmax.item()) == int(np.argmax(ref.logits[0]))
            if step == first:
                assert eng.rebuilds == 1
        tok = argmax.cpu().numpy().astype(np.int64)
    assert eng.rebuilds == expect, (eng.rebuilds, expect)
    eng.close()


def test_engine_refreshes_its_schedule_and_stays_exact():
    """Engine.step rebuilds the schedule each time a sequence has grown by a quarter of an attention split
    (the open-ended last split would otherwise take every new key): 1100 steps, exact after the first
    rebuild and at the end."""
    say("test_engine_refreshes_its_schedule_and_stays_exact: tiny engine, 1100 steps")
    _run_long(refresh_off=False)


def test_engine_rebuilds_a_stale_schedule_and_stays_exact():
    """With the refresh switched off for the first schedule, its attention splits run out of room
    after ~1000 steps; the library refuses that step, Engine.step rebuilds and issues it again."""
    say("test_engine_rebuilds_a_stale_schedule_and_stays_exact: tiny engine, 1100 steps")
    _run_long(refresh_off=True)
