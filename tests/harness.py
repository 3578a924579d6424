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
                attn_norm=synth.to_u16(lw["attn_norm"]), w_qkv=synth.to_u16(lw["w_qkv"]),
                w_o=synth.to_u16(lw["w_o"]), w_router=synth.to_u16(lw["w_router"]),
                router_bias=None if rb is None else rb.detach().cpu().numpy().astype(np.float32),
                w_gate=None, w_up=None, w_down=None)
        return self._get(("layer", l), mk)

    def expert(self, l, e):
        lw = self.w["layers"][l]
        return self._get(("expert", l, int(e)), lambda: (synth.to_u16(lw["w_gate"][int(e)]),
                                                          synth.to_u16(lw["w_up"][int(e)]),
                                                          synth.to_u16(lw["w_down"][int(e)])))

    def lm_head_rows(self, start, stop):
        return self._get(("lm", start, stop), lambda: synth.to_u16(self.w["lm_head"][start:stop]))

    def drop_layers(self):
        """Forget cached per-layer tensors (bounded host memory for long models)."""
        self._cache = {k: v for k, v in self._cache.items() if k[0] == "embed"}


def dense_weights(w):
    """Fully materialised host copy (small models)."""
    layers = []
    for lw in w["layers"]:
        rb = lw["router_bias"]
        layers.append(oracle.decode.LayerWeights(
            attn_norm=synth.to_u16(lw["attn_norm"]), w_qkv=synth.to_u16(lw["w_qkv"]),
            w_o=synth.to_u16(lw["w_o"]), w_router=synth.to_u16(lw["w_router"]),
            router_bias=None if rb is None else rb.detach().cpu().numpy().astype(np.float32),
            w_gate=synth.to_u16(lw["w_gate"]), w_up=synth.to_u16(lw["w_up"]),
            w_down=synth.to_u16(lw["w_down"])))
    return oracle.DenseWeights(embed=synth.to_u16(w["embed"]),
                               lm_head=None if w["lm_head"] is None else synth.to_u16(w["lm_head"]),
                               final_norm=synth.to_u16(w["final_norm"]), layers=layers)


def host_kv(k, v):
    return oracle.PagedKV(k=[synth.to_u16(t) for t in k], v=[synth.to_u16(t) for t in v])


def tiny_setup(wl=None, seed=0, gains="ones", batch=None, device="cpu"):
    """Generated inputs for a small workload: weights, KV, tables, lengths, first tokens."""
    wl = wl or synth.workload("tiny")
    if batch is not None:
        wl = synth.workload(wl.name, batch=batch) if wl.name in synth.WORKLOADS else wl
    bias = synth.zipf_router_bias(wl) if wl.zipf_s else None
    w = synth.make_weights(wl, seed=seed, device=device, gains=gains, router_bias=bias)
    ctx = synth.context_lengths(wl)
    bt, num_pages = synth.make_block_tables(ctx, wl.steps, wl.page_size)
    k, v = synth.make_kv(wl, num_pages, device=device)
    tokens = synth.first_tokens(wl)
    return dict(wl=wl, w=w, ctx=ctx, block_tables=bt, num_pages=num_pages, k=k, v=v, tokens=tokens)
