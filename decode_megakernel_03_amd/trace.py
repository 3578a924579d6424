"""Decode the per-task trace of a step (MK_FLAG_TRACE) into timings and a Perfetto/Chrome JSON.

Each task record is sixteen uint64: (task id | worker << 32, t_start, t_ready, t_end, mark0..11) in
100 MHz ticks of the GPU's constant real-time clock: t_ready is when its last dependency wait
ended, so t_ready - t_start is time spent waiting (with its first weight block already in flight)
and t_end - t_ready is time spent executing and signalling; marks 0..6 are op-specific phase ends
(attention: query loaded, scores, softmax + PV, partial signalled; expert slice: routing table
loaded, activations staged, GEMV done), 0 where unset. Words 11..15 are not times but
measurements: shader clock cycles over the task, then of the task's last dependency wait and its
store drain: round trip of the first poll, drain duration, round trip of the last poll (ticks) and
number of polls.
"""

import json

import numpy as np

OPS = {1: "qkv", 2: "router", 3: "gateup", 4: "attn", 5: "out", 6: "lmhead", 7: "merge"}
TICK_US = 0.01
WORDS = 16
MARKS = WORDS - 4
TIME_MARKS = 7


def decode(trace, tasks):
    """trace uint64 [n_tasks, WORDS]; tasks int32 [n_tasks, 16] (descriptors). Returns a record array."""
    t0 = trace[:, 1].min()
    rec = np.zeros(len(trace), dtype=[("id", "i4"), ("worker", "i4"), ("op", "i4"), ("layer", "i4"),
                                      ("start", "f8"), ("ready", "f8"), ("end", "f8"), ("mark", "f8", (TIME_MARKS,)), ("cycles", "f8"),
                                      ("poll_first", "f8"), ("drain", "f8"), ("poll_last", "f8"), ("polls", "i4")])
    rec["id"] = (trace[:, 0] & 0xFFFFFFFF).astype(np.int64)
    rec["worker"] = (trace[:, 0] >> 32).astype(np.int64)
    rec["op"] = tasks[:, 0]
    rec["layer"] = tasks[:, 1]
    rec["start"] = (trace[:, 1] - t0) * TICK_US
    rec["ready"] = (trace[:, 2] - t0) * TICK_US
    rec["end"] = (trace[:, 3] - t0) * TICK_US
    marks = trace[:, 4:4 + TIME_MARKS].astype(np.float64)
    rec["mark"] = np.where(marks > 0, (marks - float(t0)) * TICK_US, np.nan)
    rec["cycles"] = trace[:, 4 + TIME_MARKS].astype(np.float64)
    rec["poll_first"] = trace[:, 5 + TIME_MARKS] * TICK_US
    rec["drain"] = trace[:, 6 + TIME_MARKS] * TICK_US
    rec["poll_last"] = trace[:, 7 + TIME_MARKS] * TICK_US
    rec["polls"] = trace[:, 8 + TIME_MARKS].astype(np.int64)
    return rec


def summary(rec, n_workers):
    lines = []
    span = rec["end"].max()
    busy = np.zeros(n_workers)
    wait = np.zeros(n_workers)
    for r in rec:
        busy[r["worker"]] += r["end"] - r["ready"]
        wait[r["worker"]] += r["ready"] - r["start"]
    lines.append(f"step span {span:.1f} us; per worker: exec {busy.mean():.1f} us ({busy.mean() / span:.0%}), "
                 f"waiting {wait.mean():.1f} us, idle between tasks {span - busy.mean() - wait.mean():.1f} us")
    for op, name in OPS.items():
        m = rec["op"] == op
        if not m.any():
            continue
        r = rec[m]
        lines.append(f"  {name:7s} n={m.sum():6d}  wait {np.mean(r['ready'] - r['start']):7.2f} us  "
                     f"exec {np.mean(r['end'] - r['ready']):7.2f} us (p90 {np.percentile(r['end'] - r['ready'], 90):6.2f})")
        prev = r["ready"]
        parts = []
        for i in range(TIME_MARKS):
            mk_i = r["mark"][:, i]
            ok = ~np.isnan(mk_i)
            if ok.any():
                parts.append(f"m{i} +{np.mean(mk_i[ok] - prev[ok]):.2f}")
                prev = np.where(ok, mk_i, prev)
        if parts:
            parts.append(f"end +{np.mean(r['end'] - prev):.2f}")
            lines.append("          phases (us, cumulative steps): " + ", ".join(parts))
        lines.append(f"          last wait: first poll {np.mean(r['poll_first']):.2f} us, last poll "
                     f"{np.mean(r['poll_last']):.2f} us (p90 {np.percentile(r['poll_last'], 90):.2f}), polls "
                     f"{np.mean(r['polls']):.1f}; drain {np.mean(r['drain']):.2f} us (p90 {np.percentile(r['drain'], 90):.2f})")
    layers = sorted(set(rec["layer"].tolist()))
    lines.append("  layer  qkv_end  route_end  gateup_end  attn_end  out_end   (us from step start)")
    for l in layers[: min(len(layers), 4)] + layers[-2:]:
        r = rec[rec["layer"] == l]
        def last(op):
            x = r[r["op"] == op]
            return x["end"].max() if len(x) else float("nan")
        lines.append(f"  {l:5d} {last(1):8.1f} {last(2):10.1f} {last(3):11.1f} {last(4):9.1f} {last(5):8.1f}")
    per_layer = []
    for l in layers:
        r = rec[(rec["layer"] == l) & (rec["op"] == 5)]
        if len(r):
            per_layer.append(r["end"].max())
    if len(per_layer) > 2:
        lines.append(f"  mean layer time {np.mean(np.diff(per_layer)):.1f} us")
    return "\n".join(lines)


def fractions(rec, n_workers):
    """Where the workers' time went in a traced step: each worker's share of the step span spent
    executing tasks (dependency met -> task end), spinning on dependency counters (task start ->
    dependency met; the task's first weight block is already in flight then) and idle (between
    tasks, and after its queue ends while others still run). Also the mean layer time, the polls
    per dependency wait and the executed time of each op as a share of all executed time."""
    t0, t1 = rec["start"].min(), rec["end"].max()
    span = t1 - t0
    exec_w = np.zeros(n_workers)
    spin_w = np.zeros(n_workers)
    np.add.at(exec_w, rec["worker"], rec["end"] - rec["ready"])
    np.add.at(spin_w, rec["worker"], rec["ready"] - rec["start"])
    tot = span * n_workers
    out = {"traced_step_us": round(float(span), 1),
           "worker_exec_frac": round(float(exec_w.sum() / tot), 4),
           "worker_spin_frac": round(float(spin_w.sum() / tot), 4),
           "worker_idle_frac": round(float(1.0 - (exec_w.sum() + spin_w.sum()) / tot), 4),
           "polls_per_wait": round(float(np.mean(rec["polls"])), 2)}
    ex = rec["end"] - rec["ready"]
    out["exec_share_by_op"] = {name: round(float(ex[rec["op"] == op].sum() / ex.sum()), 4)
                               for op, name in OPS.items() if (rec["op"] == op).any()}
    ends = [rec["end"][(rec["layer"] == l) & (rec["op"] == 5)].max()
            for l in sorted(set(rec["layer"].tolist())) if ((rec["layer"] == l) & (rec["op"] == 5)).any()]
    if len(ends) > 2:
        out["mean_layer_us"] = round(float(np.mean(np.diff(ends))), 2)
    return out


def chrome_json(rec, path):
    ev = []
    for r in rec:
        name = OPS.get(int(r["op"]), str(r["op"]))
        if r["ready"] > r["start"]:
            ev.append({"name": f"wait {name}", "ph": "X", "pid": 0, "tid": int(r["worker"]), "ts": float(r["start"]),
                       "dur": float(r["ready"] - r["start"]), "args": {"layer": int(r["layer"])}})
        ev.append({"name": name, "ph": "X", "pid": 0, "tid": int(r["worker"]), "ts": float(r["ready"]),
                   "dur": float(r["end"] - r["ready"]), "args": {"layer": int(r["layer"]), "task": int(r["id"])}})
    with open(path, "w") as f:
        json.dump({"traceEvents": ev}, f)
