"""Host-side checks of libmk without a GPU: the library loads and exports every symbol the header
declares, and the static scheduler's plans are valid, deadlock-free under random interleavings
(CPU simulation of the persistent loop), and report forced stalls the way the watchdog would."""

import os
import re

import numpy as np
import pytest

from decode_megakernel_03_amd import mk, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "mk.h")).read()
    declared = set(re.findall(r"\b(mk_\w+)\s*\(", header))
    assert declared == set(mk.EXPORTED)
    for name in declared:
        assert hasattr(mk.LIB, name), name


def _desc(wl, batch, ctx_max):
    max_pages = (ctx_max + 1024 + 15) // 16
    return mk.model_desc(wl, num_pages=batch * max_pages, max_pages_per_seq=max_pages, max_batch=batch)


CASES = [
    ("tiny", [65], 512),
    ("tiny", [65, 17, 200], 512),
    ("full", [8193], 512),
    ("full", [8193] * 8, 512),
    ("full", [1025, 30000, 4096, 77, 16, 17, 32768, 9000], 512),
    ("full", [262145], 512),
    ("full", [8193], 64),
    ("layer", [8193], 512),
    ("full_fp8", [8193], 512),
    ("full_b8_fp8", [8193] * 8, 512),
    ("full_mxfp4", [8193], 512),
    ("full_b8_mxfp4", [8193] * 8, 512),
]


@pytest.mark.parametrize("flags", [0, mk.MK_FLAG_STATIC_EXPERTS], ids=["queue", "static"])
@pytest.mark.parametrize("name,lens,workers", CASES)
def test_plan_valid_and_deadlock_free(name, lens, workers, flags):
    wl = synth.workload(name)
    desc = _desc(wl, len(lens), max(lens))
    plan = mk.mk_plan_build(desc, lens, workers, flags=flags)
    try:
        st, msg = mk.mk_plan_validate(plan)
        assert st == mk.MK_OK, msg
        for seed in range(3 if wl.n_layers > 2 else 6):
            st, msg = mk.mk_plan_simulate(plan, seed)
            assert st == mk.MK_OK, msg
        info = mk.mk_plan_info_get(plan)
        assert info.n_workers == workers
        # balance: no worker carries much more than its share of the streamed bytes
        assert info.bytes_max_worker <= 1.6 * info.bytes_total / workers + 600_000
        assert info.key_capacity_min >= min(lens) + 256
    finally:
        mk.mk_plan_destroy(plan)


def test_plan_structure_full_bs1():
    """Counts per layer and the structural properties the method relies on."""
    wl = synth.workload("full")
    desc = _desc(wl, 1, 8193)
    plan = mk.mk_plan_build(desc, [8193], 512)
    tasks, qoff = mk.mk_plan_export(plan)
    mk.mk_plan_destroy(plan)
    op = tasks[:, 0]
    L = 48
    assert (op == 6).sum() == 512                                     # lm_head spread over every worker
    out_rows = tasks[op == 5][:, 3]                                   # rows of each output task
    assert out_rows.sum() == L * 2048 and out_rows.min() >= 1          # every output row once per layer
    # output rows of layer l wait on the attention merges of layer l only (every KV group's merges
    # signal the layer's attention counter, each group on sub-counters of its own)
    att = tasks[op == 4]
    out = tasks[op == 5]
    mrg = tasks[op == 7]
    for l in (0, 17, 47):
        m_l = mrg[mrg[:, 1] == l]
        o_l = out[out[:, 1] == l]
        assert len(m_l) == 4 * 4 and set(m_l[:, 12]) == set(o_l[:, 4])  # 4 slices per group
        for g in range(4):
            assert (m_l[:, 3] == g).sum() == 4
        a_l = att[att[:, 1] == l]
        assert np.all(a_l[:, 13] == -1) and np.all(a_l[:, 10] == -1)  # splits only signal arrival
        for mt in m_l:                                                # a merge waits for every split of its group
            grp = a_l[(a_l[:, 2] == mt[2]) & (a_l[:, 3] == mt[3])]
            assert mt[8] == grp[0, 12] and mt[9] == len(grp) == mt[7] and set(grp[:, 12]) == {mt[8]}
        assert np.all(o_l[:, 5] == 16)                                 # output rows wait for all 16 slices
    # a merge runs on a worker that ran one of its group's splits
    worker = np.repeat(np.arange(512), np.diff(qoff))
    for i in np.where(op == 7)[0][:64]:
        t = tasks[i]
        same = (op == 4) & (tasks[:, 1] == t[1]) & (tasks[:, 2] == t[2]) & (tasks[:, 3] == t[3])
        assert worker[i] in set(worker[same])
    # attention of group g waits only on the QKV tiles of group g (no false dependency on other groups)
    qkv = tasks[op == 1]
    for g in range(4):
        a = att[(att[:, 1] == 3) & (att[:, 3] == g)]
        producers = qkv[(qkv[:, 1] == 3) & (qkv[:, 12] == a[0, 8])]
        rows = np.concatenate([np.arange(r0, r0 + n) for r0, n in producers[:, 2:4]])
        heads = set(rows[rows < 4096] // 128)
        assert heads == set(range(8 * g, 8 * g + 8))
        assert set(rows[(rows >= 4096) & (rows < 4608)] // 128) == {32 + g}
    # router and QKV tiles never wait on anything produced in their own layer
    first = tasks[(op <= 2)]
    assert np.all(first[first[:, 1] == 0][:, 8] == -1)
    # every queue is level-ordered
    lv = tasks[:, 14]
    for w in range(512):
        q = lv[qoff[w]:qoff[w + 1]]
        assert np.all(np.diff(q) >= 0)


def test_simulated_watchdog_names_the_blocked_wait():
    wl = synth.workload("tiny")
    desc = _desc(wl, 1, 65)
    plan = mk.mk_plan_build(desc, [65], 16)
    tasks, qoff = mk.mk_plan_export(plan)
    # stall the worker that owns a router tile of layer 0 right before that tile
    rows = np.nonzero((tasks[:, 0] == 2) & (tasks[:, 1] == 0))[0]
    t = int(rows[0])
    w = int(np.searchsorted(qoff, t, side="right") - 1)
    st, msg = mk.mk_plan_simulate(plan, 1, stall_worker=w, stall_at=t - int(qoff[w]))
    mk.mk_plan_destroy(plan)
    assert st == mk.MK_ERR_DEVICE
    assert "watchdog" in msg and "waits for counter" in msg


def test_plan_rejects_bad_inputs():
    wl = synth.workload("tiny")
    desc = _desc(wl, 2, 65)
    with pytest.raises(mk.MkError):
        mk.mk_plan_build(desc, [0], 8)                 # empty sequence
    with pytest.raises(mk.MkError):
        mk.mk_plan_build(desc, [65, 65, 65], 8)        # batch above max_batch
    bad = mk.model_desc(wl, 64, 64)
    bad.page_size = 32
    with pytest.raises(mk.MkError):
        mk.mk_plan_build(bad, [65], 8)
    bad = mk.model_desc(wl, 64, 64)
    bad.hidden = 512
    with pytest.raises(mk.MkError):
        mk.mk_plan_build(bad, [65], 8)


def test_schedule_capacity_grows_with_split():
    wl = synth.workload("full")
    desc = _desc(wl, 1, 8193)
    plan = mk.mk_plan_build(desc, [8193], 512, split_keys=256)
    info = mk.mk_plan_info_get(plan)
    mk.mk_plan_destroy(plan)
    assert info.n_attn_splits == 48 * 4 * 33
    assert info.key_capacity_min == 8192 + 1024


STEAL_PROBES = 4     # sub-queues one expert task draws from (the kernel's constant)


def _drain_queue(tickets, nq, n_items, rng):
    """The expert-queue protocol of the kernel, with random interleavings of the tasks' draws: a
    draw takes the next item of one sub-queue (an atomic add on its head) and snapshots every head;
    a task draws from its own sub-queue until a draw lands past the last item, then steals from the
    sub-queue with the most items left in its last snapshot (STEAL_PROBES draws at most), and stops
    when the snapshot shows none. Returns how often each item was run."""
    heads = [0] * nq
    runs = np.zeros(n_items, dtype=int)

    def rem(snap):
        r = [max(0, -(-(n_items - (h * nq + q)) // nq)) for q, h in enumerate(snap)]
        best = max(r)
        return r.index(best) if best > 0 else -1

    state = []
    for q in tickets:
        k = heads[q]; heads[q] += 1
        state.append({"sq": q, "probes": 1, "k": k, "steal": rem(list(heads))})
    live = list(range(len(tickets)))
    while live:
        i = live[rng.integers(len(live))]
        st = state[i]
        item = st["sq"] + nq * st["k"]
        if item >= n_items:
            if st["steal"] < 0 or st["probes"] >= STEAL_PROBES:
                live.remove(i)
                continue
            st["probes"] += 1
            st["sq"] = st["steal"]
        else:
            runs[item] += 1
        st["k"] = heads[st["sq"]]; heads[st["sq"]] += 1
        st["steal"] = rem(list(heads))
    return runs


@pytest.mark.parametrize("name,lens,workers", [("full", [8193] * 8, 512), ("full", [8193, 8193], 512), ("tiny", [65, 17, 200], 16),
                                               ("full", [1025, 30000, 4096, 77, 16, 17, 32768, 9000], 512),
                                               ("full_fp8", [8193] * 8, 512), ("full_mxfp4", [8193] * 8, 512)])
def test_expert_queue_runs_every_item_once(name, lens, workers):
    """Queue-mode expert tasks (batches above 1): one queue counter per layer that nothing waits on, every sub-queue
    owned by some task, and under random interleavings every (slot, slice) item of the step's union
    is run exactly once whatever the union size."""
    wl = synth.workload(name)
    desc = _desc(wl, len(lens), max(lens))
    plan = mk.mk_plan_build(desc, lens, workers)
    tasks, qoff = mk.mk_plan_export(plan)
    mk.mk_plan_destroy(plan)
    gu = tasks[(tasks[:, 0] == 3) & (tasks[:, 1] == 1)]
    assert len(gu) <= workers
    qc, nq, slices, nfs = gu[0, 5], gu[0, 3], gu[0, 4], gu[0, 6]
    assert np.all(gu[:, 5] == qc) and np.all(gu[:, 3] == nq) and set(gu[:, 2]) == set(range(nq))
    assert slices * nfs >= wl.expert_ffn > (slices - 1) * nfs
    assert not np.isin(tasks[:, [8, 10, 12, 13]], [qc]).any()
    rng = np.random.default_rng(0)
    slots = min(wl.n_experts, wl.top_k * len(lens))
    for nu in sorted({wl.top_k, (wl.top_k + slots) // 2, slots}):
        # the kernel's item size: three adjacent slices per draw (two for MXFP4 rows) once there
        # are 4 slices per worker
        gmax = 2 if wl.weights == "mxfp4" else 3
        grain = gmax if nu * slices >= 4 * workers and gmax * nfs <= 48 else 1
        slices_c = -(-slices // grain)
        runs = _drain_queue(list(gu[:, 2]), nq, nu * slices_c, rng)
        assert np.all(runs == 1)
        # the items of a slot cover its FFN rows exactly once
        rows = np.zeros(wl.expert_ffn, dtype=int)
        for j in range(slices_c):
            f0 = j * grain * nfs
            rows[f0:min(wl.expert_ffn, f0 + grain * nfs)] += 1
        assert np.all(rows == 1)


def test_batch1_keeps_static_expert_slices():
    """At batch 1 the union is always top_k experts: the slices are dealt statically."""
    wl = synth.workload("full")
    plan = mk.mk_plan_build(_desc(wl, 1, 8193), [8193], 512)
    tasks, _ = mk.mk_plan_export(plan)
    mk.mk_plan_destroy(plan)
    gu = tasks[tasks[:, 0] == 3]
    assert np.all(gu[:, 5] == -1) and len(gu) == 48 * 8 * len(set(gu[gu[:, 1] == 0][:, 3]))


def test_stream_read_bandwidth_rejects_bad_arguments():
    """The measurement helper validates its arguments before touching the GPU."""
    for args in ((0, 1 << 20, 1), (16 + 4, 1 << 20, 1), (1 << 20, 8, 1), (1 << 20, 1 << 20, 0)):
        with pytest.raises(mk.MkError) as e:
            mk.mk_stream_read_bandwidth(*args)
        assert e.value.status == mk.MK_ERR_INVALID_ARG


CHUNKED = [
    ("tiny", [5, 6, 7, 8], 4, 64),                                   # one sequence, 4 consecutive positions
    ("tiny", [40, 61, 62, 63, 64, 65, 17], 4, 512),                  # decode rows mixed with a 4-row chunk
    ("full", list(range(4001, 4009)), 8, 512),                       # a whole step of one prompt
    ("full", [8193, 300, 301, 302, 303, 304, 305, 17], 6, 512),      # mixed: decode rows and a 6-row chunk
]


@pytest.mark.parametrize("name,lens,rows,workers", CHUNKED)
def test_chunked_plan_publishes_kv_in_the_qkv_tasks(name, lens, rows, workers):
    """Schedules for rows of one sequence in one step: valid and deadlock-free, every K tile one whole
    head (RoPE pairs dims d and d + D/2) and every V tile whole groups of 8 dims (16-byte stores),
    and the host's capacity leaves room for steps that advance a row by `rows` positions."""
    wl = synth.workload(name)
    desc = _desc(wl, len(lens), max(lens) + 8 * 64)
    plan = mk.mk_plan_build(desc, lens, workers, rows_per_seq=rows)
    try:
        st, msg = mk.mk_plan_validate(plan)
        assert st == mk.MK_OK, msg
        for seed in range(3):
            st, msg = mk.mk_plan_simulate(plan, seed)
            assert st == mk.MK_OK, msg
        tasks, _ = mk.mk_plan_export(plan)
        D, HQ, HKV = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        qkv = tasks[tasks[:, 0] == 1]                          # OP_QKV: a0 first row, a1 rows
        k = qkv[(qkv[:, 2] >= HQ * D) & (qkv[:, 2] < (HQ + HKV) * D)]
        v = qkv[qkv[:, 2] >= (HQ + HKV) * D]
        assert len(k) == wl.n_layers * HKV and np.all(k[:, 3] == D) and np.all((k[:, 2] - HQ * D) % D == 0)
        assert np.all(v[:, 3] % 8 == 0) and np.all(v[:, 2] % 8 == 0)
        assert mk.mk_plan_info_get(plan).key_capacity_min >= min(lens) + 32 * rows
    finally:
        mk.mk_plan_destroy(plan)


@pytest.mark.parametrize("name,lens", [("full", [8193]), ("full", [8193] * 8), ("tiny", [65])])
def test_plan_info_reports_its_split_length(name, lens):
    """mk_plan_info.split_keys is the split the plan uses: the attention tasks of a sequence cover
    split_keys keys each, except the open-ended last one."""
    wl = synth.workload(name)
    desc = _desc(wl, len(lens), max(lens))
    plan = mk.mk_plan_build(desc, lens, 512)
    try:
        info = mk.mk_plan_info_get(plan)
        tasks, _ = mk.mk_plan_export(plan)
    finally:
        mk.mk_plan_destroy(plan)
    att = tasks[tasks[:, 0] == 4]
    closed = att[att[:, 5] >= 0]
    assert info.split_keys >= 16 and info.split_keys % 16 == 0
    assert len(closed) == 0 or (closed[:, 5] - closed[:, 4] == info.split_keys).all()
