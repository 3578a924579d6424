"""Thin ctypes binding over libmk.so (the C ABI declared in include/mk.h).

Functions carry the ABI's names and only marshal arguments: every step of the decode path runs
in the library's HIP kernel. Importing this module loads libmk.so and raises if it is missing -
there is no fallback path. ``Engine`` is a convenience owner of an engine handle that keeps the
torch tensors it points at alive.
"""

import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK, MK_ERR_INVALID_ARG, MK_ERR_UNSUPPORTED, MK_ERR_HIP, MK_ERR_OOM = 0, -1, -2, -3, -4
MK_ERR_NO_SCHEDULE, MK_ERR_SCHEDULE_STALE, MK_ERR_DEVICE = -5, -6, -7
MK_ABI_VERSION = 3
MK_WEIGHTS_BF16 = 0
MK_WEIGHTS_FP8 = 1
MK_WEIGHTS_MXFP4 = 2
_WEIGHT_FORMATS = {"bf16": MK_WEIGHTS_BF16, "fp8": MK_WEIGHTS_FP8, "mxfp4": MK_WEIGHTS_MXFP4}
MK_MAX_BATCH = 8
MK_FLAG_TRACE = 1
MK_FLAG_NO_PREFETCH = 2
MK_FLAG_STATIC_EXPERTS = 4
MK_FLAG_OPROJ_PER_GROUP = 8
DESC_WORDS = 16

EXPORTED = ["mk_create", "mk_set_options", "mk_build_schedule", "mk_build_schedule_chunked", "mk_prefill",
            "mk_decode_step", "mk_set_step_outputs",
            "mk_sync", "mk_get_error", "mk_reset", "mk_destroy", "mk_plan_build", "mk_plan_info_get",
            "mk_plan_export", "mk_plan_validate", "mk_plan_simulate", "mk_engine_plan", "mk_plan_destroy",
            "mk_stream_read_bandwidth", "mk_handoff_litmus", "mk_handoff_litmus_noalloc",
            "mk_server_create", "mk_server_submit", "mk_server_pause", "mk_server_resume", "mk_server_run",
            "mk_server_wait", "mk_server_poll", "mk_server_take", "mk_server_stats", "mk_server_last_step",
            "mk_server_get_error", "mk_server_destroy"]


# bound at import: during interpreter shutdown the module globals (sys among them) may already be None
_finalizing = sys.is_finalizing


class MkError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libmk status {status}: {msg}")
        self.status = status


class ModelDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "expert_ffn", "vocab", "page_size", "num_pages", "max_batch", "max_pages_per_seq", "has_router_bias",
        "has_lm_head")] + [("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("weight_format", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class WeightPtrs(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("w_qkv", _PP), ("w_o", _PP), ("w_router", _PP), ("router_bias", _PP),
                ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP), ("k_cache", _PP), ("v_cache", _PP)]


class Options(ctypes.Structure):
    _fields_ = [("workers_per_cu", ctypes.c_int32), ("split_keys", ctypes.c_int32),
                ("watchdog_ms", ctypes.c_int32), ("flags", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_int32), ("n_workers", ctypes.c_int32), ("n_counters", ctypes.c_int32),
                ("max_queue", ctypes.c_int32), ("bytes_total", ctypes.c_int64), ("bytes_max_worker", ctypes.c_int64),
                ("n_attn_splits", ctypes.c_int32), ("key_capacity_min", ctypes.c_int32),
                ("split_keys", ctypes.c_int32)]


class ServerConfig(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("start_held", ctypes.c_int32), ("topk_out", ctypes.c_void_p),
                ("router_logits_out", ctypes.c_void_p), ("hidden_out", ctypes.c_void_p), ("logits_out", ctypes.c_void_p)]


class Request(ctypes.Structure):
    _fields_ = [("request_id", ctypes.c_int64), ("prompt_len", ctypes.c_int32), ("first_token", ctypes.c_int32),
                ("max_new_tokens", ctypes.c_int32), ("n_pages", ctypes.c_int32), ("pages", ctypes.POINTER(ctypes.c_int32)),
                ("prompt", ctypes.POINTER(ctypes.c_int32))]


class ServerStep(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("batch", ctypes.c_int32), ("rebuilt", ctypes.c_int32),
                ("request_id", ctypes.c_int64 * MK_MAX_BATCH), ("position", ctypes.c_int32 * MK_MAX_BATCH),
                ("token_in", ctypes.c_int32 * MK_MAX_BATCH), ("token_out", ctypes.c_int32 * MK_MAX_BATCH),
                ("prefill_rows", ctypes.c_int32)]


class ServerStats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("tokens", ctypes.c_int64), ("rebuilds", ctypes.c_int64),
                ("active", ctypes.c_int32), ("pending", ctypes.c_int32), ("finished", ctypes.c_int32),
                ("paused", ctypes.c_int32), ("busy_seconds", ctypes.c_double), ("prefill_tokens", ctypes.c_int64)]


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m decode_megakernel_03_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    P32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "mk_create": [ctypes.POINTER(ModelDesc), ctypes.POINTER(WeightPtrs), ctypes.POINTER(vp)],
        "mk_set_options": [vp, ctypes.POINTER(Options)],
        "mk_build_schedule": [vp, i32, P32],
        "mk_build_schedule_chunked": [vp, i32, P32, i32],
        "mk_prefill": [vp, P32, i32, i32, P32, vp, vp, vp],
        "mk_decode_step": [vp, vp, vp, vp, vp, vp, vp],
        "mk_set_step_outputs": [vp, vp, vp, vp, vp, vp],
        "mk_sync": [vp],
        "mk_get_error": [vp, ctypes.c_char_p, sz],
        "mk_reset": [vp],
        "mk_destroy": [vp],
        "mk_plan_build": [ctypes.POINTER(ModelDesc), i32, P32, i32, i32, ctypes.c_uint32, i32, ctypes.POINTER(vp)],
        "mk_plan_info_get": [vp, ctypes.POINTER(PlanInfo)],
        "mk_plan_export": [vp, P32, P32],
        "mk_plan_validate": [vp, ctypes.c_char_p, sz],
        "mk_plan_simulate": [vp, u64, i32, i32, ctypes.c_char_p, sz],
        "mk_engine_plan": [vp],
        "mk_plan_destroy": [vp],
        "mk_stream_read_bandwidth": [vp, sz, i32, ctypes.POINTER(ctypes.c_double)],
        "mk_handoff_litmus": [i32, i32, i32, ctypes.POINTER(u64), ctypes.POINTER(u64)],
        "mk_handoff_litmus_noalloc": [i32, i32, i32, ctypes.POINTER(u64), ctypes.POINTER(u64)],
        "mk_server_create": [vp, ctypes.POINTER(ServerConfig), ctypes.POINTER(vp)],
        "mk_server_submit": [vp, ctypes.POINTER(Request)],
        "mk_server_pause": [vp], "mk_server_resume": [vp], "mk_server_run": [vp, ctypes.c_int64],
        "mk_server_wait": [vp],
        "mk_server_poll": [vp, ctypes.POINTER(ctypes.c_int64), P32, i32],
        "mk_server_take": [vp, ctypes.c_int64, P32, i32, P32],
        "mk_server_stats": [vp, ctypes.POINTER(ServerStats)],
        "mk_server_last_step": [vp, ctypes.POINTER(ServerStep), ctypes.POINTER(vp)],
        "mk_server_get_error": [vp, ctypes.c_char_p, sz],
        "mk_server_destroy": [vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = None if name in ("mk_destroy", "mk_plan_destroy") else (vp if name == "mk_engine_plan" else ctypes.c_int)
    return lib


# torch brings its own HIP and HSA runtimes, libmk.so links the system ROCm ones; the process works
# with both only when torch's are loaded first (loading libmk.so first left mk_create without a HIP
# device once torch had initialised the GPU), so torch is imported before the library is loaded
import torch  # noqa: E402,F401

# MK_LIBRARY names another build of the same C ABI (e.g. to compare two builds in one process tree)
LIB = load(os.environ.get("MK_LIBRARY", LIB_PATH))


def _i32_array(values):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def model_desc(wl, num_pages, max_pages_per_seq, max_batch=None, has_router_bias=False):
    """mk_model_desc for a workload description (decode_megakernel_03_amd.synth.Workload)."""
    return ModelDesc(MK_ABI_VERSION, wl.n_layers, wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                     wl.n_experts, wl.top_k, wl.expert_ffn, wl.vocab, wl.page_size, int(num_pages),
                     int(max_batch or wl.batch), int(max_pages_per_seq), int(bool(has_router_bias)),
                     int(bool(wl.lm_head)), float(wl.rope_theta), float(wl.rms_eps),
                     _WEIGHT_FORMATS[getattr(wl, "weights", "bf16")])


# ---------------------------------------------------------------- same-name wrappers

def _check(status, handle=None, what=""):
    if status != MK_OK:
        msg = what
        if handle:
            buf = ctypes.create_string_buffer(1024)
            LIB.mk_get_error(handle, buf, 1024)
            msg = f"{what}: {buf.value.decode()}"
        raise MkError(status, msg)


def mk_create(desc, ptrs):
    h = ctypes.c_void_p()
    _check(LIB.mk_create(ctypes.byref(desc), ctypes.byref(ptrs), ctypes.byref(h)), None, "mk_create")
    return h


def mk_set_options(h, workers_per_cu=0, split_keys=0, watchdog_ms=0, flags=0):
    _check(LIB.mk_set_options(h, ctypes.byref(Options(workers_per_cu, split_keys, watchdog_ms, flags))), h, "mk_set_options")


def mk_build_schedule(h, seq_lens):
    arr = _i32_array(seq_lens)
    _check(LIB.mk_build_schedule(h, len(seq_lens), arr), h, "mk_build_schedule")


def mk_build_schedule_chunked(h, seq_lens, rows_per_seq):
    arr = _i32_array(seq_lens)
    _check(LIB.mk_build_schedule_chunked(h, len(seq_lens), arr, int(rows_per_seq)), h, "mk_build_schedule_chunked")


def mk_prefill(h, tokens, start, block_table, logits_out=None, topk_out=None, stream=None):
    """Positions [start, start + len(tokens)) of one sequence through the decode kernel (host token and
    block-table arrays; optional device outputs: last position's logits [V], routed experts [L, n, k])."""
    _check(LIB.mk_prefill(h, _i32_array(tokens), len(tokens), int(start), _i32_array(block_table), _ptr(logits_out),
                          _ptr(topk_out), ctypes.c_void_p(stream or 0)), h, "mk_prefill")


def mk_decode_step(h, tokens, positions, block_tables, seq_lens, logits_out, stream=None):
    st = LIB.mk_decode_step(h, _ptr(tokens), _ptr(positions), _ptr(block_tables), _ptr(seq_lens), _ptr(logits_out),
                            ctypes.c_void_p(stream or 0))
    return st


def mk_set_step_outputs(h, argmax_out=None, topk_out=None, hidden_out=None, trace_out=None, router_logits_out=None):
    _check(LIB.mk_set_step_outputs(h, _ptr(argmax_out), _ptr(topk_out), _ptr(hidden_out), _ptr(trace_out),
                                   _ptr(router_logits_out)), h, "mk_set_step_outputs")


def mk_sync(h):
    return LIB.mk_sync(h)


def mk_get_error(h):
    buf = ctypes.create_string_buffer(2048)
    st = LIB.mk_get_error(h, buf, 2048)
    return st, buf.value.decode()


def mk_reset(h):
    _check(LIB.mk_reset(h), h, "mk_reset")


def mk_destroy(h):
    LIB.mk_destroy(h)


def mk_stream_read_bandwidth(buf_ptr, nbytes, reps=5):
    """Streaming-read bandwidth (bytes/s) of the current device over a caller-owned device buffer."""
    out = ctypes.c_double(0.0)
    _check(LIB.mk_stream_read_bandwidth(ctypes.c_void_p(buf_ptr), ctypes.c_size_t(nbytes), int(reps), ctypes.byref(out)),
           None, "mk_stream_read_bandwidth")
    return out.value


def mk_handoff_litmus(rounds, words, workgroups):
    """Hand-off protocol self-test; returns (status, stale words, words checked)."""
    stale, checked = ctypes.c_uint64(0), ctypes.c_uint64(0)
    st = LIB.mk_handoff_litmus(int(rounds), int(words), int(workgroups), ctypes.byref(stale), ctypes.byref(checked))
    return st, stale.value, checked.value


MK_LITMUS_NOALLOC_MAX_WORDS = 16384


def mk_handoff_litmus_noalloc(rounds, words, workgroups):
    """The allocation-free form of mk_handoff_litmus (fixed device scratch array); (status, stale, checked)."""
    stale, checked = ctypes.c_uint64(0), ctypes.c_uint64(0)
    st = LIB.mk_handoff_litmus_noalloc(int(rounds), int(words), int(workgroups), ctypes.byref(stale), ctypes.byref(checked))
    return st, stale.value, checked.value


def mk_plan_build(desc, seq_lens, n_workers, split_keys=0, flags=0, rows_per_seq=1):
    h = ctypes.c_void_p()
    _check(LIB.mk_plan_build(ctypes.byref(desc), len(seq_lens), _i32_array(seq_lens), int(n_workers),
                             int(split_keys), int(flags), int(rows_per_seq), ctypes.byref(h)), None, "mk_plan_build")
    return h


def mk_plan_info_get(plan):
    info = PlanInfo()
    _check(LIB.mk_plan_info_get(plan, ctypes.byref(info)), None, "mk_plan_info_get")
    return info


def mk_plan_export(plan):
    import numpy as np
    info = mk_plan_info_get(plan)
    tasks = np.zeros((info.n_tasks, DESC_WORDS), np.int32)
    qoff = np.zeros(info.n_workers + 1, np.int32)
    P32 = ctypes.POINTER(ctypes.c_int32)
    _check(LIB.mk_plan_export(plan, tasks.ctypes.data_as(P32), qoff.ctypes.data_as(P32)), None, "mk_plan_export")
    return tasks, qoff


def mk_plan_validate(plan):
    buf = ctypes.create_string_buffer(1024)
    return LIB.mk_plan_validate(plan, buf, 1024), buf.value.decode()


def mk_plan_simulate(plan, seed, stall_worker=-1, stall_at=0):
    buf = ctypes.create_string_buffer(1024)
    return LIB.mk_plan_simulate(plan, int(seed), int(stall_worker), int(stall_at), buf, 1024), buf.value.decode()


def mk_engine_plan(h):
    return ctypes.c_void_p(LIB.mk_engine_plan(h))


def mk_plan_destroy(plan):
    LIB.mk_plan_destroy(plan)


# ---------------------------------------------------------------- convenience owner

class Engine:
    """Owns an engine over torch-resident weights (dict from synth.make_weights) and KV caches."""

    def __init__(self, wl, weights, k_cache, v_cache, num_pages, max_pages_per_seq, max_batch=None):
        self.wl = wl
        self._keep = (weights, k_cache, v_cache)
        L = wl.n_layers
        has_bias = weights["layers"][0]["router_bias"] is not None
        self.desc = model_desc(wl, num_pages, max_pages_per_seq, max_batch, has_bias)

        def arr(key):
            a = (ctypes.c_void_p * L)(*[weights["layers"][l][key].data_ptr() for l in range(L)])
            return ctypes.cast(a, _PP), a

        keep = []
        fields = {}
        for key in ("attn_norm", "w_qkv", "w_o", "w_router", "w_gate", "w_up", "w_down"):
            p, a = arr(key)
            fields[key] = p
            keep.append(a)
        rb = None
        if has_bias:
            a = (ctypes.c_void_p * L)(*[weights["layers"][l]["router_bias"].data_ptr() for l in range(L)])
            rb = ctypes.cast(a, _PP)
            keep.append(a)
        ka = (ctypes.c_void_p * L)(*[t.data_ptr() for t in k_cache])
        va = (ctypes.c_void_p * L)(*[t.data_ptr() for t in v_cache])
        keep += [ka, va]
        ptrs = WeightPtrs(weights["embed"].data_ptr(),
                          0 if weights["lm_head"] is None else weights["lm_head"].data_ptr(),
                          weights["final_norm"].data_ptr(), fields["attn_norm"], fields["w_qkv"], fields["w_o"],
                          fields["w_router"], rb, fields["w_gate"], fields["w_up"], fields["w_down"],
                          ctypes.cast(ka, _PP), ctypes.cast(va, _PP))
        self.h = mk_create(self.desc, ptrs)
        self._ptr_arrays = keep

    def set_options(self, **kw):
        mk_set_options(self.h, **kw)

    def build_schedule(self, seq_lens, rows_per_seq=1):
        """Schedule for the batch's current lengths; rows_per_seq > 1 when one sequence holds several
        rows (consecutive positions) of a step."""
        mk_build_schedule_chunked(self.h, list(seq_lens), rows_per_seq)
        self._lens = [int(v) for v in seq_lens]
        self._growth = int(rows_per_seq)
        self._steps = 0
        self.rebuilds = 0
        # keys a sequence may grow past these lengths before the step rebuilds the schedule
        self.refresh_keys = max(1, self.plan_info().split_keys // 4)

    def prefill(self, tokens, start, block_table, logits_out=None, topk_out=None, stream=None):
        """Chunked prefill of one sequence (mk_prefill); the engine has no schedule afterwards."""
        mk_prefill(self.h, tokens, start, block_table, logits_out, topk_out, stream)
        self._lens = None

    def set_step_outputs(self, **kw):
        self._outs = kw
        mk_set_step_outputs(self.h, **kw)

    def step(self, tokens, positions, block_tables, seq_lens, logits_out, stream=None):
        """One decode step. Every sequence grows by one token per step, and the keys past the lengths
        the schedule was built for land in each sequence's open-ended last attention split: once a
        sequence has grown by refresh_keys (a quarter of a split) the schedule is rebuilt for the step's
        lengths (given as a tensor: one host read then). When a sequence would outgrow the splits'
        capacity the library refuses the step before launching it (MK_ERR_SCHEDULE_STALE); the
        schedule is then rebuilt for the current lengths and the step is issued again."""
        if (getattr(self, "_lens", None) is not None and hasattr(seq_lens, "cpu")
                and self._steps * self._growth >= self.refresh_keys):
            lens = seq_lens.cpu().tolist()
            if max(n - b for n, b in zip(lens, self._lens)) >= self.refresh_keys:
                rebuilds = self.rebuilds
                self.build_schedule(lens, self._growth)
                self.rebuilds = rebuilds + 1
        st = mk_decode_step(self.h, tokens, positions, block_tables, seq_lens, logits_out, stream)
        if st == MK_ERR_SCHEDULE_STALE and getattr(self, "_lens", None) is not None:
            # the step's own lengths (rows of one sequence advance by several positions per step)
            lens = seq_lens.cpu().tolist() if hasattr(seq_lens, "cpu") else [n + self._steps for n in self._lens]
            rebuilds = self.rebuilds
            self.build_schedule(lens, self._growth)
            self.rebuilds = rebuilds + 1
            st = mk_decode_step(self.h, tokens, positions, block_tables, seq_lens, logits_out, stream)
        if st != MK_OK:
            _check(st, self.h, "mk_decode_step")
        self._steps += 1

    def sync(self):
        st = mk_sync(self.h)
        if st != MK_OK:
            _check(st, self.h, "mk_sync")

    def error(self):
        return mk_get_error(self.h)

    def plan_info(self):
        return mk_plan_info_get(mk_engine_plan(self.h))

    def close(self):
        if getattr(self, "h", None):
            mk_destroy(self.h)
            self.h = None

    def __del__(self, _finalizing=_finalizing):
        # at interpreter shutdown the HIP runtime (and a profiler attached to it) may already be torn
        # down: leave the engine to process exit then, and never call into the library. (The check is
        # bound as a default argument: module globals may already be cleared when this runs.)
        if not getattr(self, "h", None) or _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- the serving loop's decode owner

def _server_check(h, st, what):
    if st != MK_OK:
        buf = ctypes.create_string_buffer(1024)
        LIB.mk_server_get_error(h, buf, 1024)
        raise MkError(st, f"{what}: {buf.value.decode()}")


def mk_server_create(engine_h, max_batch, start_held=False, topk_out=None, router_logits_out=None, hidden_out=None,
                     logits_out=None):
    cfg = ServerConfig(int(max_batch), int(bool(start_held)), _ptr(topk_out).value, _ptr(router_logits_out).value,
                       _ptr(hidden_out).value, _ptr(logits_out).value)
    h = ctypes.c_void_p()
    _check(LIB.mk_server_create(engine_h, ctypes.byref(cfg), ctypes.byref(h)), engine_h, "mk_server_create")
    return h


def mk_server_submit(h, request_id, pages, prompt_len, first_token, max_new_tokens, prompt=None):
    """Queue a sequence: prefilled elsewhere (prompt None: K/V of [0, prompt_len) in its pages, first_token
    decoded at prompt_len), or with its prompt tokens, which the server prefills itself."""
    arr = _i32_array(pages)
    pr = None if prompt is None else _i32_array(prompt)
    if pr is not None:
        prompt_len, first_token = len(prompt), 0
    req = Request(int(request_id), int(prompt_len), int(first_token), int(max_new_tokens), len(pages),
                  ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)),
                  None if pr is None else ctypes.cast(pr, ctypes.POINTER(ctypes.c_int32)))
    _server_check(h, LIB.mk_server_submit(h, ctypes.byref(req)), "mk_server_submit")


def mk_server_pause(h):
    _server_check(h, LIB.mk_server_pause(h), "mk_server_pause")


def mk_server_resume(h):
    _server_check(h, LIB.mk_server_resume(h), "mk_server_resume")


def mk_server_run(h, n_steps):
    _server_check(h, LIB.mk_server_run(h, int(n_steps)), "mk_server_run")


def mk_server_wait(h):
    _server_check(h, LIB.mk_server_wait(h), "mk_server_wait")


def mk_server_poll(h, max_items=64):
    ids = (ctypes.c_int64 * max_items)()
    nt = (ctypes.c_int32 * max_items)()
    n = LIB.mk_server_poll(h, ids, nt, max_items)
    if n < 0:
        raise MkError(MK_ERR_INVALID_ARG, "mk_server_poll")
    return [(int(ids[i]), int(nt[i])) for i in range(n)]


def mk_server_take(h, request_id, cap=1 << 16):
    buf = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32(0)
    _server_check(h, LIB.mk_server_take(h, int(request_id), buf, cap, ctypes.byref(n)), "mk_server_take")
    return [int(buf[i]) for i in range(n.value)]


def mk_server_stats(h):
    st = ServerStats()
    _server_check(h, LIB.mk_server_stats(h, ctypes.byref(st)), "mk_server_stats")
    return st


def mk_server_last_step(h):
    rec = ServerStep()
    lp = ctypes.c_void_p()
    _server_check(h, LIB.mk_server_last_step(h, ctypes.byref(rec), ctypes.byref(lp)), "mk_server_last_step")
    B = rec.batch
    return {"step": rec.step, "batch": B, "rebuilt": bool(rec.rebuilt),
            "request_id": list(rec.request_id[:B]), "position": list(rec.position[:B]),
            "token_in": list(rec.token_in[:B]), "token_out": list(rec.token_out[:B]), "logits_ptr": lp.value,
            "prefill_rows": rec.prefill_rows}


def mk_server_get_error(h):
    buf = ctypes.create_string_buffer(1024)
    st = LIB.mk_server_get_error(h, buf, 1024)
    return st, buf.value.decode()


def mk_server_destroy(h):
    return LIB.mk_server_destroy(h)
