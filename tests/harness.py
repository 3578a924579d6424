"""Glue between the seeded generator (decode_megakernel_03_amd.synth) and the CPU oracle.

Test infrastructure: used by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg.
It converts generated torch tensors (host or device) into the oracle's uint16 bf16 arrays, lazily
for device-resident weights so that the oracle only copies the tensors it touches.
"""

import numpy as np

import oracle
from decode_megakernel_03_amd import synth


def dims_of(wl):
    return oracle.Dims(n_layers=wl.n_layers, hidden=wl.hidden, n_q_heads=wl.n_q_heads,
                       n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim, n_experts=wl.n_experts,
                       top_k=wl.top_k, expert_ffn=wl.expert_ffn,
                       vocab=wl.vocab if wl.lm_head else 0, page_size=wl.page_size,
                       rope_theta=wl.rope_theta, rms_eps=wl.rms_eps)


def host_matrix(w, t):
    """A generated matrix as the oracle reads it: ``synth.to_host``, and packed MXFP4 rows wrapped as
    ``oracle.mxfp4.Mxfp4Rows`` (their K follows from the row length)."""
    a = synth.to_host(t)
    if w.get("format") == "mxfp4":
        return oracle.mxfp4.Mxfp4Rows(a, oracle.mxfp4.k_of_row_bytes(a.shape[-1]))
    return a


class LazyWeights:
    """Oracle weight provider over generated torch tensors; copies to host on first touch."""

    def __init__(self, w):
        self.w = w
        self._cache = {}
        self.final_norm = synth.to_u16(w["final_norm"])

    def _get(self, key, fn):
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    def embed_row(self, token):
        return self._get(("embed", int(token)), lambda: synth.to_u16(self.w["embed"][int(token)]))

    def layer(self, l):
        def mk():
            lw = self.w["layers"][l]
            rb = lw["router_bias"]
            return oracle.decode.LayerWeights(
                attn_norm=synth.to_u16(lw["attn_norm"]), w_qkv=host_matrix(self.w, lw["w_qkv"]),
                w_o=host_matrix(self.w, lw["w_o"]), w_router=host_matrix(self.w, lw["w_router"]),
                router_bias=None if rb is None else rb.detach().cpu().numpy().astype(np.float32),
                w_gate=None, w_up=None, w_down=None)
        return self._get(("layer", l), mk)

    def expert(self, l, e):
        lw = self.w["layers"][l]
        return self._get(("expert", l, int(e)), lambda: (host_matrix(self.w, lw["w_gate"][int(e)]),
                                                          host_matrix(self.w, lw["w_up"][int(e)]),
                                                          host_matrix(self.w, lw["w_down"][int(e)])))

    def lm_head_rows(self, start, stop):
        return self._get(("lm", start, stop), lambda: host_matrix(self.w, self.w["lm_head"][start:stop]))

    def drop_layers(self):
        """Forget cached per-layer tensors (bounded host memory for long models)."""
        self._cache = {k: v for k, v in self._cache.items() if k[0] == "embed"}


def dense_weights(w):
    """Fully materialised host copy (small models)."""
    layers = []
    for lw in w["layers"]:
        rb = lw["router_bias"]
        layers.append(oracle.decode.LayerWeights(
            attn_norm=synth.to_u16(lw["attn_norm"]), w_qkv=host_matrix(w, lw["w_qkv"]),
            w_o=host_matrix(w, lw["w_o"]), w_router=host_matrix(w, lw["w_router"]),
            router_bias=None if rb is None else rb.detach().cpu().numpy().astype(np.float32),
            w_gate=host_matrix(w, lw["w_gate"]), w_up=host_matrix(w, lw["w_up"]),
            w_down=host_matrix(w, lw["w_down"])))
    return oracle.DenseWeights(embed=synth.to_u16(w["embed"]),
                               lm_head=None if w["lm_head"] is None else host_matrix(w, w["lm_head"]),
                               final_norm=synth.to_u16(w["final_norm"]), layers=layers)


def host_kv(k, v):
    return oracle.PagedKV(k=[synth.to_u16(t) for t in k], v=[synth.to_u16(t) for t in v])


def tiny_setup(wl=None, seed=0, gains="ones", batch=None, device="cpu", ctx=None):
    """Generated inputs for a small workload: weights, KV, tables, lengths, first tokens.
    ``ctx`` overrides the prefilled context per sequence (e.g. 0: the sequence's first token)."""
    wl = wl or synth.workload("tiny")
    if batch is not None:
        wl = synth.workload(wl.name, batch=batch) if wl.name in synth.WORKLOADS else wl
    bias = synth.zipf_router_bias(wl) if wl.zipf_s else None
    w = synth.make_weights(wl, seed=seed, device=device, gains=gains, router_bias=bias)
    ctx = synth.context_lengths(wl) if ctx is None else np.asarray(ctx, np.int64)
    bt, num_pages = synth.make_block_tables(ctx, wl.steps, wl.page_size)
    k, v = synth.make_kv(wl, num_pages, device=device)
    tokens = synth.first_tokens(wl)
    return dict(wl=wl, w=w, ctx=ctx, block_tables=bt, num_pages=num_pages, k=k, v=v, tokens=tokens)


class RoutingMismatch(AssertionError):
    """The GPU took a routing decision the oracle does not accept as a near-tie."""

    def __init__(self, msg, ref, forced):
        super().__init__(msg)
        self.ref, self.forced = ref, forced


def replay_near_ties(run, g_topk, near_tie, max_rounds=32):
    """Reconcile the GPU's expert sets g_topk [L, B, k] with the oracle, layer by layer.

    ``run(forced)`` runs the oracle step with ``forced_topk=forced`` and returns its result. The
    first layer where the two disagree must be a near-tie for every disagreeing token: oracle margin
    r_(k) - r_(k+1) <= near_tie, and the GPU's set is the oracle's with its rank-k expert replaced by
    its rank-(k+1) expert (ranks from a stable sort of the oracle's router logits); the oracle is then rerun with the GPU's sets forced
    there, which changes everything after that layer, and the walk continues. Disagreements after
    an unreplayed flip are never judged against an oracle that has already diverged.
    Returns (result, forced); raises RoutingMismatch otherwise.
    """
    forced = {}
    L, B = g_topk.shape[:2]
    for _ in range(max_rounds):
        ref = run(forced or None)
        for l in range(L):
            diff = [b for b in range(B)
                    if (l, b) not in forced and set(g_topk[l, b].tolist()) != set(ref.topk[l, b].tolist())]
            if diff:
                break
        else:
            return ref, forced
        for b in diff:
            gs, rs = set(g_topk[l, b].tolist()), set(ref.topk[l, b].tolist())
            k = len(rs)
            # the oracle's ranking of this token's router logits (ties -> lower index, as route())
            order = np.argsort(-np.asarray(ref.router_logits[l, b]), kind="stable")
            swap = (rs - gs == {int(order[k - 1])}) and (gs - rs == {int(order[k])})
            if not (ref.margin[l, b] <= near_tie and swap):
                raise RoutingMismatch(f"layer {l} token {b}: GPU experts {sorted(gs)} != oracle {sorted(rs)} "
                                      f"(oracle ranks k, k+1 = {int(order[k - 1])}, {int(order[k])}; margin "
                                      f"{ref.margin[l, b]:.3g}; earlier near-tie replays {sorted(forced)})",
                                      ref, forced)
            forced[(l, b)] = sorted(gs)
    raise RoutingMismatch(f"more than {max_rounds} rounds of near-tie replays", ref, forced)


def bf16_step_mismatch(g16, h16, floor=1e-5):
    """Mask of entries where two bf16 arrays (uint16 patterns) differ by more than one bf16 step.

    A K/V entry is an fp32 result rounded to bf16; two fp32 results that differ by reduction order
    round to the same bf16 or to neighbours, so entries may differ by at most the spacing of bf16
    at the larger of the two magnitudes (2^(floor(log2|v|) - 7)). Differences up to ``floor`` in
    absolute value are accepted as well: the fp32 values themselves may differ by that much (rounding
    noise near zero; after many layers, the deviation their inputs carry)."""
    gd = oracle.bf16_to_f32(np.asarray(g16, np.uint16)).astype(np.float64)
    hd = oracle.bf16_to_f32(np.asarray(h16, np.uint16)).astype(np.float64)
    mag = np.maximum(np.abs(gd), np.abs(hd))
    with np.errstate(divide="ignore"):
        step = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    diff = np.abs(gd - hd)
    return diff > step + floor


def check_full_step(dims, lw, kv0, tokens, positions, block_tables, g_topk, g_rlog, g_logits, g_argmax, near_tie,
                    router_tol, max_abs=2e-2, max_rel=5e-3, g_kv=None, kv_floor=None):
    """Gates of one GPU decode step against the oracle run on the same inputs (teacher-forced: the
    oracle starts from kv0, the KV cache as the step began). Routing: bit-exact up to near-ties
    (replayed); router logits |d| <= router_tol up to the first replay; logits max |d| and relative L2 per
    token; greedy tokens equal. With g_kv (a function (layer, page, slot) -> (k16, v16) of the GPU's
    cache after the step) the new K/V rows are compared too (one bf16 step + kv_floor). Returns stats."""
    import copy
    kv_last = {}

    def run(forced):
        kv = copy.deepcopy(kv0)
        kv_last["kv"] = kv
        return oracle.decode_step(dims, lw, kv, np.asarray(tokens, np.int64), np.asarray(positions, np.int64),
                                  block_tables, np.asarray(positions, np.int64) + 1, forced_topk=forced)

    ref, replay = replay_near_ties(run, g_topk, near_tie)
    L, B = g_topk.shape[:2]
    first = min([l for l, _ in replay], default=L)
    dr = float(np.abs(g_rlog.astype(np.float64) - ref.router_logits)[:first].max()) if first else 0.0
    assert dr <= router_tol, f"router logits max|d| {dr:.3g} > {router_tol}"
    stats = {"router_logits_maxabs": dr, "near_ties": len(replay), "min_margin": float(ref.margin.min())}
    for b in range(B):
        d = np.abs(g_logits[b].astype(np.float64) - ref.logits[b]).max()
        rel = np.linalg.norm(g_logits[b].astype(np.float64) - ref.logits[b]) / np.linalg.norm(ref.logits[b])
        stats["logits_maxabs"] = max(stats.get("logits_maxabs", 0.0), float(d))
        stats["logits_rel"] = max(stats.get("logits_rel", 0.0), float(rel))
        assert d <= max_abs and rel <= max_rel, f"token {b}: logits max|d| {d:.3g} rel {rel:.3g}"
    assert np.array_equal(np.asarray(g_argmax), np.argmax(ref.logits, 1)), "greedy tokens differ"
    if g_kv is not None:
        kvo = kv_last["kv"]
        nbad = ndiff = ntot = 0
        for b in range(B):
            p_b = int(positions[b])
            page, slot = int(block_tables[b][p_b // dims.page_size]), p_b % dims.page_size
            for l in range(L):
                gk, gv = g_kv(l, page, slot)
                for g16, h16 in ((gk, kvo.k[l][page, :, slot, :]), (gv, kvo.v[l][page, :, slot, :])):
                    nbad += int(bf16_step_mismatch(g16, h16, floor=kv_floor).sum())
                    ndiff += int((g16 != h16).sum())
                    ntot += g16.size
        stats["kv_rows_differ"] = f"{ndiff}/{ntot}"
        assert nbad == 0 and ndiff <= max(2, ntot // 50), f"new K/V rows: {nbad} beyond tolerance, {ndiff}/{ntot} differ"
    return stats
