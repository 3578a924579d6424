"""The oracle's prefill: the plain definition of writing a prompt's K/V, as one causal forward pass.

Test infrastructure only (see the package docstring for who may import it).

What the pages fix
------------------
* The pages' engine prefills with ordinary (PyTorch) kernels and uses the megakernel for decode
  only (P2 body; P3 "Limitations and Future Plans"); prefill in the megakernel, and batches that
  mix prefill and decode, are the pages' next step (P3, same section).
* A prefill computes, for every prompt position, what a decode step at that position computes:
  the same layers (``oracle.decode``'s docstring, readings R1-R10), with each position attending to
  the keys at or before it.

Formulation
-----------
The whole prompt at once, in matrix form: every projection is one product over all n positions,
attention is a masked n x T score matrix per head (query i sees key j iff j <= start + i), and
each expert runs on the block of positions routed to it. This is a second formulation of the same
definition, apart from ``decode_step`` (one position at a time); the tests pin the two against each
other, against a split prompt, and against causality. Keys and values are rounded to bf16 and
written before attending (R6), so every position reads its own and its predecessors' keys in the
rounded form, exactly as a decode step at that position would.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .bf16 import f32_to_bf16, f64_to_bf16
from .decode import _dec, gather_paged, rope_cos_sin, route, silu


@dataclass
class PrefillResult:
    logits: Optional[np.ndarray]     # float32 [n, V] (all positions) or [V] (last only); None without lm_head
    x_final: np.ndarray              # [n, H] residual stream after the last layer
    topk: np.ndarray                 # int32 [L, n, k] selected experts, ascending index
    router_logits: np.ndarray        # [L, n, E]
    margin: np.ndarray               # [L, n] r_(k) - r_(k+1) of the sorted logits


def _rmsnorm_rows(x, gain, eps, dtype):
    """R1 for every row of x [n, H]."""
    ms = np.mean(x * x, axis=1, dtype=dtype, keepdims=True)
    return (x / np.sqrt(ms + dtype(eps))) * gain


def _rope_rows(x, pos, theta, dtype):
    """R3 for x [n, heads, D] with row i at position pos[i] (rotate-half pairing)."""
    d = x.shape[-1]
    cs = [rope_cos_sin(int(p), d, theta, dtype) for p in pos]
    c = np.stack([a for a, _ in cs])[:, None, :]          # [n, 1, D/2]
    s = np.stack([b for _, b in cs])[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def prefill(dims, w, kv, tokens, block_table, start=0, dtype=np.float32, forced_topk=None, all_logits=False,
            lm_head_chunk=8192):
    """Positions [start, start + n) of one sequence whose keys and values for positions < start are
    already in the paged cache ``kv`` (mutated: the prompt's K/V are written at their positions).

    ``forced_topk`` maps (layer, i) -> experts for position start + i (replay of a near-tied routing
    decision, as in ``decode_step``). Returns the logits of the last position (or of all when
    ``all_logits``), the final residual stream, and the routing of every layer and position.
    """
    L, H, D = dims.n_layers, dims.hidden, dims.head_dim
    hq, hkv, K, E = dims.n_q_heads, dims.n_kv_heads, dims.top_k, dims.n_experts
    grp = hq // hkv
    n = len(tokens)
    pos = start + np.arange(n)
    T = start + n
    enc = f32_to_bf16 if dtype == np.float32 else f64_to_bf16
    topk = np.zeros((L, n, K), np.int32)
    rlog = np.zeros((L, n, E), dtype)
    margin = np.zeros((L, n), np.float64)
    # causal mask over the cached keys 0..T-1: query i sees key j iff j <= start + i
    visible = np.arange(T)[None, :] <= pos[:, None]        # [n, T]

    x = np.stack([_dec(w.embed_row(int(t)), dtype) for t in tokens])   # [n, H]
    for l in range(L):
        lw = w.layer(l)
        nrm = _rmsnorm_rows(x, _dec(lw.attn_norm, dtype), dims.rms_eps, dtype)
        # attention branch: all positions' q, k, v in one product
        qkv = nrm @ _dec(lw.w_qkv, dtype).T                                   # [n, QKVR]
        q = _rope_rows(qkv[:, : hq * D].reshape(n, hq, D), pos, dims.rope_theta, dtype)
        k_new = _rope_rows(qkv[:, hq * D: (hq + hkv) * D].reshape(n, hkv, D), pos, dims.rope_theta, dtype)
        v_new = qkv[:, (hq + hkv) * D:].reshape(n, hkv, D)
        for i in range(n):
            page = int(block_table[int(pos[i]) // dims.page_size])
            slot = int(pos[i]) % dims.page_size
            kv.k[l][page, :, slot, :] = enc(k_new[i])
            kv.v[l][page, :, slot, :] = enc(v_new[i])
        kk = _dec(gather_paged(kv.k[l], block_table, T, dims.page_size), dtype)   # [T, Hkv, D]
        vv = _dec(gather_paged(kv.v[l], block_table, T, dims.page_size), dtype)
        o = np.empty((n, hq, D), dtype)
        for h in range(hq):
            g = h // grp
            s = (q[:, h, :] @ kk[:, g, :].T) / np.sqrt(dtype(D))               # [n, T]
            s = np.where(visible, s, dtype(-np.inf))
            p = np.exp(s - np.max(s, axis=1, keepdims=True))
            o[:, h, :] = (p @ vv[:, g, :]) / np.sum(p, axis=1, dtype=dtype, keepdims=True)
        attn = o.reshape(n, hq * D) @ _dec(lw.w_o, dtype).T                   # [n, H]
        # MoE branch from the same normed input (R2): route every position, then each expert once
        # over the positions routed to it, adding in ascending expert index (R8)
        r = nrm @ _dec(lw.w_router, dtype).T
        if lw.router_bias is not None:
            r = r + lw.router_bias.astype(dtype)
        wsel = np.zeros((n, E), dtype)
        for i in range(n):
            sel, wt, mg = route(r[i], K)
            if forced_topk is not None and (l, i) in forced_topk:
                sel = np.sort(np.asarray(forced_topk[(l, i)], dtype=np.int32))
                rs = r[i][sel]
                e = np.exp(rs - np.max(rs))
                wt = e / np.sum(e, dtype=dtype)
            topk[l, i], margin[l, i] = sel, mg
            wsel[i, sel] = wt
        rlog[l] = r
        moe = np.zeros((n, H), dtype)
        for e_id in np.unique(topk[l]):
            rows = np.nonzero(np.any(topk[l] == e_id, axis=1))[0]
            g_, u_, d_ = w.expert(l, int(e_id))
            a = nrm[rows]
            hmid = silu(a @ _dec(g_, dtype).T) * (a @ _dec(u_, dtype).T)           # [m, F]
            moe[rows] += wsel[rows, e_id][:, None] * (hmid @ _dec(d_, dtype).T)
        x = (x + attn) + moe

    logits = None
    if dims.vocab > 0:
        nf = _rmsnorm_rows(x if all_logits else x[-1:], _dec(w.final_norm, dtype), dims.rms_eps, dtype)
        logits = np.empty((nf.shape[0], dims.vocab), np.float32)
        for s0 in range(0, dims.vocab, lm_head_chunk):
            s1 = min(dims.vocab, s0 + lm_head_chunk)
            logits[:, s0:s1] = (nf @ _dec(w.lm_head_rows(s0, s1), dtype).T).astype(np.float32)
        if not all_logits:
            logits = logits[0]
    return PrefillResult(logits, x, topk, rlog, margin)
