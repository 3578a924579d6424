#!/usr/bin/env python3
"""Decode throughput of the persistent megakernel on one MI355X.

A step is one decode step of the synthetic 48-layer parallel-MoE model (hidden 2048, 32/4 heads of
128, 128 experts top-8, FFN 768, vocab 151936, random bf16 weights) for the batch, with the KV cache
resident in HBM. Greedy decoding runs on the device (each step's argmax is the next step's token).

Prints ONE JSON line: tok/s, % of HBM speed of light (algorithmic bytes / step time / 8 TB/s, with
the expert union measured from the step's routing), the roofline of the step kernel, and the CPU
oracle timed on the host cores over one full decode step (which also checks the first GPU step).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

_WEIGHTS_DESC = {"bf16": "bf16 weights and KV",
                 "fp8": "FP8 E4M3 matrices with per-row scales, bf16 embedding, norms and KV",
                 "mxfp4": "MXFP4 matrices (E2M1, E8M0 scale per 32), bf16 embedding, norms and KV"}
PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
METRIC = "decode tok/s on 1 GPU at bs1 & bs8, 8K ctx; % of HBM speed-of-light"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_host.cpp", "mk_internal.h"):    # the kernel and its schedule
        h.update(open(os.path.join(ROOT, "decode_megakernel_03_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="full")
    ap.add_argument("--batch", type=int, default=0)
    ap.add_argument("--context", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers-per-cu", type=int, default=0)
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--refresh-keys", type=int, default=-1,
                    help="rebuild the schedule once a sequence has grown this many keys past the lengths it was "
                         "built for (-1: a quarter of an attention split, as the engine does; 0: only when stale)")
    ap.add_argument("--no-b8", action="store_true", help="with the default workload, skip the batch-8 line in the JSON")
    ap.add_argument("--trace", default="", help="write the traced step's summary (.txt) here")
    ap.add_argument("--trace-records", action="store_true", help="with --trace, also write the records (.npy) and a Chrome JSON")
    ap.add_argument("--no-trace-stats", action="store_true", help="skip the traced step after timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling the HBM write counter)")
    ap.add_argument("--read-calibration", action="store_true",
                    help="only stream 1 GiB with the library's read kernel, 3 dispatches (for scaling the HBM "
                         "read counter: the same 16-byte non-temporal loads as the step kernel)")
    return ap.parse_args()


def read_calibration():
    import torch
    from decode_megakernel_03_amd import mk
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    bw = mk.mk_stream_read_bandwidth(a.data_ptr(), n, 2)     # one untimed pass + 2 timed: 3 dispatches
    torch.cuda.synchronize()
    del a
    torch.cuda.empty_cache()
    print(json.dumps({"read_bytes_per_dispatch": n, "dispatches": 3, "bandwidth_gb_s": round(bw / 1e9, 1)}))


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        return copy_calibration()
    if args.read_calibration:
        return read_calibration()
    from decode_megakernel_03_amd import metrics, mk, synth

    if args.workload == "prefill":
        return bench_prefill(args)
    if args.workload == "serve":
        return bench_serve(args)
    over = {}
    if args.batch:
        over["batch"] = args.batch
    if args.context:
        over["context"] = args.context
    wl = synth.workload(args.workload, **over)
    B = wl.batch
    want_cpu = not args.no_cpu_baseline
    r = measure(wl, args, args.steps, args.warmup, keep_kv_host=want_cpu)
    eng, info, ctx, bt_np, w = r["eng"], r["info"], r["ctx"], r["bt_np"], r["w"]
    step_ms, span_ms, tok_s, achieved, sol_frac = r["step_ms"], r["span_ms"], r["tok_s"], r["achieved"], r["sol_frac"]
    timed_bytes, union, topk_h, logits0, tok0, kv_host0 = r["timed_bytes"], r["union"], r["topk_h"], r["logits0"], r["tok0"], r["kv_host0"]
    tokens, pos_all, bt, len_all, logits, h, total_steps = r["loop"]
    # where the workers' time goes (executing / spinning on counters / idle), from one traced step
    # after the timed ones (tracing adds a little time per task, so it is kept out of the timing)
    sched = None
    if not args.no_trace_stats:
        sched = run_trace(args, eng, tokens, pos_all, bt, len_all, logits, h, total_steps, args.trace)

    traffic = None
    prof = os.path.join(ROOT, "profiles", f"traffic_{wl.name}_b{B}.json")
    if os.path.exists(prof):
        rec = json.load(open(prof))
        if rec.get("kernel_hash") == kernel_source_hash():
            # measured HBM bytes per launch over the same per-launch duration as `achieved`
            traffic = round(rec["bytes_per_launch"] / float(np.mean(step_ms / 1e3)) / 1e9, 1)

    cpu = None
    parity = None
    if want_cpu:
        cpu, parity = cpu_baseline(wl, w, kv_host0, tok0.cpu().numpy(), ctx, bt_np, logits0, topk_h[0])
    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(span_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.n_layers}-layer parallel-MoE decoder, batch {B}, context {int(ctx.max())}"
                               f"{' (ragged)' if wl.ragged else ''}, {_WEIGHTS_DESC[wl.weights]}, fp32 arithmetic",
                   "batch": B, "context": int(ctx.max()), "layers": wl.n_layers, "hidden": wl.hidden,
                   "experts": f"{wl.n_experts} top-{wl.top_k}", "vocab": wl.vocab,
                   "workers": info.n_workers, "tasks_per_step": info.n_tasks},
        "sol_fraction": round(sol_frac, 4),
        "bytes_per_step": int(timed_bytes.mean()),
        "experts_union_mean": round(float(union[args.warmup:].mean()), 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "parity_first_step": parity,
        "schedule": sched,
        "schedule_rebuilds_in_timed_steps": len([s for s in r["rebuilds"] if s >= args.warmup]),
    }
    # release the engine and every device buffer of this workload now, while the runtime (and any
    # profiler attached to it) is up, instead of leaving them to interpreter shutdown
    eng.close()
    del r, w, eng, tokens, pos_all, bt, len_all, logits, kv_host0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # the metric is quoted at batch 1 and batch 8: the batch-8 figure of the same model and context
    # joins the line (its own engine, inputs and timing; value above stays the batch-1 workload)
    if args.workload == "full" and args.batch in (0, 1) and not args.no_b8:
        wl8 = synth.workload("full_b8")
        r8 = measure(wl8, args, 16, 4)
        sched8 = None
        if not args.no_trace_stats:
            sched8 = run_trace(args, r8["eng"], *r8["loop"], path=(args.trace + "_b8") if args.trace else "")
        r8["eng"].close()
        r8["eng"] = r8["w"] = r8["loop"] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["bs8"] = {"workload": f"{wl8.name}: batch 8, context {int(r8['ctx'].max())} each",
                      "value": round(r8["tok_s"], 2), "unit": "tok/s", "steps": 16, "warmup": 4,
                      "ms_per_step": round(r8["span_ms"] / 16, 4), "sol_fraction": round(r8["sol_frac"], 4),
                      "bytes_per_step": int(r8["timed_bytes"].mean()),
                      "experts_union_mean": round(float(r8["union"][4:].mean()), 2),
                      "roofline_frac": round(r8["achieved"] / PEAK_HBM, 4), "schedule": sched8}
        del r8
    # the measured streaming-read ceiling of this machine, next to the 8 TB/s figure
    ceil = read_ceiling()
    out["hbm_read_ceiling"] = {"value": round(ceil / 1e9, 1), "unit": "GB/s",
                               "method": "mk_stream_read_bandwidth: 4 GiB streamed 5 times after one warm-up pass"}
    out["roofline"]["frac_of_read_ceiling"] = round(achieved / ceil, 4)
    print(json.dumps(out), flush=True)
    torch.cuda.synchronize()


def bench_prefill(args):
    """Prompt positions per second through mk_prefill (chunks of 8 consecutive positions per step of the
    decode kernel) on the 48-layer model, one prompt of --context positions (default 2048) from
    position 0. Bytes per chunk step: dense weights, the union of the chunk's routed experts, lm_head
    and the sequence's K/V once (the rows of a chunk read the same keys)."""
    import torch
    from decode_megakernel_03_amd import metrics, mk, synth
    P = args.context or 2048
    wl = synth.workload("full", context=P)
    log(f"[bench] prefill: generating the 48-layer model; prompt of {P} positions")
    w = synth.make_weights(wl, seed=0, device="cuda")
    npg = (P + wl.page_size - 1) // wl.page_size
    k, v = synth.make_kv(wl, npg, device="cuda")
    eng = mk.Engine(wl, w, k, v, npg, npg, max_batch=8)
    prompt = np.random.default_rng(31).integers(0, wl.vocab, P).tolist()
    bt = list(range(npg))
    logits = torch.zeros(wl.vocab, dtype=torch.float32, device="cuda")
    topk = torch.zeros(wl.n_layers, P, wl.top_k, dtype=torch.int32, device="cuda")
    eng.prefill(prompt[:64], 0, bt, logits_out=logits)          # warm-up (untimed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    eng.prefill(prompt, 0, bt, logits_out=logits, topk_out=topk)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eng.sync()
    th = topk.cpu().numpy()
    total = 0
    for c0 in range(0, P, 8):
        c1 = min(P, c0 + 8)
        union = [len(np.unique(th[l, c0:c1])) for l in range(wl.n_layers)]
        total += metrics.weight_bytes(synth.workload("full", batch=c1 - c0), union) + metrics.kv_bytes(wl, [c1])
    rate = P / wall
    achieved = total / wall
    log(f"[bench] prefill: {P} positions in {wall:.3f} s -> {rate:.1f} positions/s; {total / 1e9:.1f} GB -> "
        f"{achieved / 1e9:.0f} GB/s ({achieved / PEAK_HBM:.1%} of 8 TB/s)")
    out = {"metric": "prefill positions/s on 1 GPU (chunks of 8 through the decode kernel)", "value": round(rate, 2),
           "unit": "positions/s", "n_gpus": 1, "steps": (P + 7) // 8, "warmup": 1, "ms_per_step": round(wall * 1e3 / ((P + 7) // 8), 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"prefill: 48-layer parallel-MoE decoder, one prompt of {P} positions from position 0, "
                                  "bf16 weights and KV, fp32 arithmetic", "prompt": P, "layers": wl.n_layers},
           "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM, 4), "traffic": None,
                        "note": "wall time of mk_prefill: schedule builds included"},
           "cpu_baseline": None, "bytes_total": int(total)}
    eng.close()
    print(json.dumps(out), flush=True)


def bench_serve(args):
    """The serving loop on the 48-layer model: requests that carry their prompts (log-uniform 64..2048
    positions, 32..256 new tokens) through the C++ decode owner with eight rows; prompts are prefilled
    in chunks that share steps with decoding sequences. Reports generated and prompt tokens per second
    of wall time (schedule rebuilds included) and the owner's step statistics."""
    import torch
    from decode_megakernel_03_amd import mk, serve, synth
    n_req = max(8, args.steps // 4) if args.steps != 128 else 32
    wl = synth.workload("full_b8")
    log(f"[bench] serve: generating the 48-layer model; {n_req} requests")
    w = synth.make_weights(wl, seed=0, device="cuda")
    reqs = synth.synthetic_prompts(wl, seed=41, n=n_req, ctx=(64, 2048), new_tokens=(32, 256))
    max_pages = max((len(p) - 1 + o + 15) // 16 for p, o in reqs)
    num_pages = 8 * max_pages
    k, v = synth.make_kv(wl, num_pages, device="cuda")
    eng = mk.Engine(wl, w, k, v, num_pages, max_pages, max_batch=8)
    srv = serve.Server(eng, 8)
    ctl = serve.ControlLoop(srv, serve.PagePool(range(num_pages)), reqs, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctl.start()
    ctl.join(timeout=900)
    wall = time.perf_counter() - t0
    st = srv.stats()
    srv.close()
    eng.close()
    gen = int(st.tokens)
    log(f"[bench] serve: {n_req} requests in {wall:.2f} s: {gen} generated ({gen / wall:.1f} tok/s), {st.prefill_tokens} "
        f"prompt positions; {st.steps} steps, {st.rebuilds} schedule rebuilds, owner busy {st.busy_seconds:.2f} s")
    out = {"metric": "serving: generated tok/s on 1 GPU (continuous batching, mixed prefill/decode)",
           "value": round(gen / wall, 2), "unit": "tok/s", "n_gpus": 1, "steps": int(st.steps), "warmup": 0,
           "ms_per_step": round(st.busy_seconds * 1e3 / max(1, st.steps), 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"serve: 48-layer parallel-MoE decoder, {n_req} requests, prompts log-uniform 64..2048, "
                                  "32..256 new tokens, 8 rows, prompts prefilled by the server", "requests": n_req},
           "prompt_positions_per_s": round(st.prefill_tokens / wall, 2),
           "total_positions_per_s": round((gen + st.prefill_tokens) / wall, 2),
           "schedule_rebuilds": int(st.rebuilds), "owner_busy_s": round(st.busy_seconds, 3), "wall_s": round(wall, 3),
           "roofline": None, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def read_ceiling(nbytes=4 << 30, reps=5):
    """Plain streaming-read bandwidth of the GPU: the library's streaming-read kernel (16-byte
    non-temporal loads on every CU) over a 4 GiB buffer, timed with HIP events."""
    import torch
    from decode_megakernel_03_amd import mk
    torch.cuda.empty_cache()
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    torch.cuda.synchronize()
    bw = mk.mk_stream_read_bandwidth(x.data_ptr(), nbytes, reps)
    del x
    torch.cuda.empty_cache()
    log(f"[bench] streaming-read ceiling: {bw / 1e9:.0f} GB/s")
    return bw


def measure(wl, args, steps, warmup, keep_kv_host=False):
    """Synthetic inputs of workload wl on the GPU, an engine and its schedule, then `warmup` untimed
    and `steps` timed decode steps (HIP events on the launch stream around every step)."""
    import torch
    from decode_megakernel_03_amd import metrics, mk, synth
    B = wl.batch
    total_steps = warmup + steps
    dev = "cuda"
    t0 = time.time()
    log(f"[bench] generating {wl.name}: {wl.n_layers} layers, batch {B}, context {wl.context} on the GPU")
    bias = synth.zipf_router_bias(wl) if wl.zipf_s else None
    w = synth.make_weights(wl, seed=0, device=dev, router_bias=bias)
    ctx = synth.context_lengths(wl)
    bt_np, num_pages = synth.make_block_tables(ctx, total_steps + 1, wl.page_size)
    k, v = synth.make_kv(wl, num_pages, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; KV pages {num_pages}")
    kv_host0 = None
    if keep_kv_host:
        from tests import harness
        kv_host0 = harness.host_kv(k, v)            # KV state before the first step (oracle input)

    eng = mk.Engine(wl, w, k, v, num_pages, bt_np.shape[1], max_batch=B)
    eng.set_options(workers_per_cu=args.workers_per_cu, split_keys=args.split_keys, flags=args.flags)
    eng.build_schedule((ctx + 1).tolist())
    info = eng.plan_info()
    log(f"[bench] schedule: {info.n_tasks} tasks on {info.n_workers} workers, {info.n_attn_splits} attention splits")

    # per-step inputs precomputed on the device: positions / lengths advance by one each step and the
    # token buffer doubles as the argmax output, so the timed loop is nothing but kernel launches
    pos_all = torch.from_numpy((ctx[None, :] + np.arange(total_steps)[:, None]).astype(np.int32)).to(dev)
    len_all = pos_all + 1
    bt = torch.from_numpy(bt_np).to(dev)
    tokens = torch.from_numpy(synth.first_tokens(wl)).to(dev)
    tok0 = tokens.clone()
    topk = torch.zeros(total_steps, wl.n_layers, B, wl.top_k, dtype=torch.int32, device=dev)
    logits = torch.empty(B, wl.vocab, dtype=torch.float32, device=dev)
    logits0 = None
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    rebuilds = []
    built_at = 0
    refresh = args.refresh_keys if args.refresh_keys >= 0 else eng.refresh_keys
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(total_steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(total_steps)]
    for s in range(total_steps):
        mk.mk_set_step_outputs(eng.h, argmax_out=tokens, topk_out=topk[s])
        if s == warmup:
            torch.cuda.synchronize()
            log(f"[bench] warmup done ({warmup} steps); timing {steps} steps")
            t_wall = time.perf_counter()
        if refresh > 0 and s > 0 and s - built_at >= refresh:
            # the open-ended last attention split has absorbed refresh_keys new keys per sequence:
            # rebuild for the current lengths (host work inside the timed region)
            mk.mk_build_schedule(eng.h, (ctx + 1 + s).tolist())
            rebuilds.append(s)
            built_at = s
        starts[s].record(stream)
        st = mk.mk_decode_step(eng.h, tokens, pos_all[s], bt, len_all[s], logits, h)
        if st == mk.MK_ERR_SCHEDULE_STALE:
            # a sequence outgrew the attention splits' room: rebuild for the current lengths (host
            # work inside the timed region, as a serving loop would pay it) and issue the step again
            mk.mk_build_schedule(eng.h, (ctx + 1 + s).tolist())
            rebuilds.append(s)
            built_at = s
            log(f"[bench] step {s}: schedule rebuilt for lengths {(ctx + 1 + s).tolist()[:4]}")
            st = mk.mk_decode_step(eng.h, tokens, pos_all[s], bt, len_all[s], logits, h)
        ends[s].record(stream)
        if st != mk.MK_OK:
            raise mk.MkError(st, mk.mk_get_error(eng.h)[1])
        if s == 0:
            torch.cuda.synchronize()
            eng.sync()
            logits0 = logits.cpu().numpy().copy()
            log("[bench] step 0 ok")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    eng.sync()
    step_ms = np.array([starts[s].elapsed_time(ends[s]) for s in range(warmup, total_steps)])
    # timed region: first start event to last end event (includes launch gaps)
    span_ms = starts[warmup].elapsed_time(ends[total_steps - 1])
    topk_h = topk.cpu().numpy()
    union = np.array([[len(np.unique(topk_h[s, l])) for l in range(wl.n_layers)] for s in range(total_steps)])
    step_bytes = np.array([metrics.step_bytes(wl, union[s], ctx + 1 + s) for s in range(total_steps)])
    timed_bytes = step_bytes[warmup:]
    tok_s = B * steps / (span_ms / 1e3)
    achieved = float(np.mean(timed_bytes / (step_ms / 1e3)))      # per launch: bytes / kernel duration
    sol_frac = float(np.sum(timed_bytes) / (span_ms / 1e3) / PEAK_HBM)
    log(f"[bench] {wl.name}: {steps} steps: mean {step_ms.mean():.3f} ms, median {np.median(step_ms):.3f} ms, "
        f"span {span_ms:.1f} ms, wall {wall * 1e3:.1f} ms -> {tok_s:.1f} tok/s; {timed_bytes.mean() / 1e9:.3f} GB/step; "
        f"{achieved / 1e9:.0f} GB/s per launch ({achieved / PEAK_HBM:.1%} of 8 TB/s)")
    return {"eng": eng, "info": info, "ctx": ctx, "bt_np": bt_np, "w": w, "step_ms": step_ms, "span_ms": span_ms,
            "tok_s": tok_s, "achieved": achieved, "sol_frac": sol_frac, "timed_bytes": timed_bytes, "union": union,
            "topk_h": topk_h, "logits0": logits0, "tok0": tok0, "kv_host0": kv_host0, "rebuilds": rebuilds,
            "loop": (tokens, pos_all, bt, len_all, logits, h, total_steps)}


def run_trace(args, eng, tokens, pos_all, bt, len_all, logits, h, total_steps, path=""):
    """One more step with per-task timestamps (after an untimed traced warm-up step): returns the
    time shares of trace.fractions; with `path`, also writes the text summary, the records and a
    Chrome JSON there."""
    import torch
    from decode_megakernel_03_amd import mk, trace
    info = eng.plan_info()
    buf = torch.zeros(info.n_tasks, trace.WORDS, dtype=torch.int64, device="cuda")
    mk.mk_set_options(eng.h, flags=args.flags | mk.MK_FLAG_TRACE)
    mk.mk_set_step_outputs(eng.h, argmax_out=tokens, trace_out=buf)
    s = total_steps - 1
    for _ in range(2):          # the second traced step is the one reported
        st = mk.mk_decode_step(eng.h, tokens, pos_all[s], bt, len_all[s], logits, h)
        if st != mk.MK_OK:
            raise mk.MkError(st, mk.mk_get_error(eng.h)[1])
        torch.cuda.synchronize()
    eng.sync()
    mk.mk_set_options(eng.h, flags=args.flags)
    mk.mk_set_step_outputs(eng.h, argmax_out=tokens)
    tr = buf.cpu().numpy().view(np.uint64)
    del buf
    tasks, qoff = mk.mk_plan_export(mk.mk_engine_plan(eng.h))
    rec = trace.decode(tr, tasks)
    summ = trace.summary(rec, info.n_workers)
    log(summ)
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path + ".txt", "w") as f:
            f.write(summ + "\n")
        if args.trace_records:
            np.save(path + ".npy", rec)
            trace.chrome_json(rec, path + ".json")
    return trace.fractions(rec, info.n_workers)


def cpu_baseline(wl, w, kv0, tokens, ctx, bt, logits_gpu, topk_gpu):
    """The oracle (numpy, fp32) on one full decode step of the same workload, on the host cores.
    Weights touched by the step are copied to the host first (an untimed pass fills the cache)."""
    import oracle
    from tests import harness
    import copy as cp
    cores = len(os.sched_getaffinity(0))
    dims = harness.dims_of(wl)
    lw = harness.LazyWeights(w)
    log(f"[bench] cpu baseline: untimed oracle pass (fetching touched weights to the host), {cores} cores")
    t = time.perf_counter()
    r = oracle.decode_step(dims, lw, cp.deepcopy(kv0), tokens, ctx, bt, ctx + 1)
    log(f"[bench] cpu baseline: fetch pass {time.perf_counter() - t:.1f}s; timed pass")
    t = time.perf_counter()
    r = oracle.decode_step(dims, lw, cp.deepcopy(kv0), tokens, ctx, bt, ctx + 1)
    dt = time.perf_counter() - t
    log(f"[bench] cpu baseline: {dt:.2f}s per step")
    d = np.abs(logits_gpu.astype(np.float64) - r.logits)
    rel = float(np.linalg.norm(logits_gpu - r.logits) / np.linalg.norm(r.logits))
    same_topk = int(sum(set(topk_gpu[l, b]) == set(r.topk[l, b]) for l in range(wl.n_layers) for b in range(wl.batch)))
    parity = {"max_abs_logit_diff": float(d.max()), "rel_l2": rel,
              "argmax_equal": bool(np.array_equal(np.argmax(logits_gpu, 1), np.argmax(r.logits, 1))),
              "topk_sets_equal": f"{same_topk}/{wl.n_layers * wl.batch}",
              "min_router_margin": float(r.margin.min())}
    cpu = {"value": round(wl.batch / dt, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
           "sample": f"one full decode step (batch {wl.batch}, {wl.n_layers} layers, context {int(ctx.max())}) "
                     f"after an untimed pass that copies the touched weights to the host"}
    return cpu, parity


if __name__ == "__main__":
    main()
