"""The oracle's decode step: the plain definition of what the megakernel computes.

Test infrastructure only (see the package docstring for who may import it).

What the pages fix
------------------
* One decode step runs the whole forward pass for a batch of at most 8 sequences (P1 "One
  persistent kernel for the whole decode step"; P2 body: batch size up to 8).
* Layers are *parallel*: attention and the MoE read the same normalized input and are rejoined
  by a residual add followed by RMSNorm (P1 "One persistent kernel for the whole decode step").
* The MoE activates a fraction of the parameters per token (P1 lede: 30B total, 3.3B active);
  the expert FFN multiplies SiLU(gate) by up ("SiLU-multiply", P3 "Key Technologies and
  Architecture"); RoPE is applied to queries and keys (same section).
* Attention reads a paged KV cache through per-sequence block tables, with ragged sequence
  lengths in one batch (P1 "From demo to a full serving system"; P3 "Key Technologies").
* Weights and KV cache are BF16 (P1 "Decode is a bandwidth game"; P2 body). The FP8 variant
  (P3 "Limitations and Future Plans" names FP8/FP4 kernels as the next step) stores the matrices
  as E4M3 codes with a float32 scale per row (``oracle.fp8``); the step is the same over the
  dequantized weights; likewise the MXFP4 variant (``oracle.mxfp4``: E2M1 codes in blocks of 32
  sharing a power-of-two scale).

Readings (the pages are silent; each is the plainest choice the rest supports)
-------------------------------------------------------------------------------
R1  RMSNorm n = x / sqrt(mean(x^2) + eps) * g with eps = 1e-6 and a per-layer gain g; a final
    RMSNorm with its own gain precedes lm_head.
R2  One input norm per layer shared by both branches; x_{l+1} = (x_l + attn) + moe; no post-norms.
R3  RoPE: rotate-half pairing (dim i with dim i + D/2), full head dim, inv_freq_i = theta^(-2i/D);
    angles pos * inv_freq formed in float64, cos/sin rounded to the working precision.
R4  GQA: query head h reads KV head h // (Hq / Hkv).
R5  Scores are q.k / sqrt(D); no bias, softcap, window, sinks or QK-norm; linears are bias-free
    except an optional per-layer router bias.
R6  The new token's K (after RoPE) and V are rounded to bf16 and written to slot ``pos`` of the
    cache *before* attending; attention covers keys [0, seq_len), the new one included, so the
    new key also scores itself in its rounded form. positions[b] == seq_lens[b] - 1.
R7  Router: r = W_r n (+ bias); the k selected experts are the k largest raw logits, ties broken
    towards the lower expert index; their weights are the softmax over the k selected logits.
    No shared expert, no capacity limit.
R8  Expert FFN: h = SiLU(W_gate n) * (W_up n), y = W_down h, with SiLU(z) = z * sigmoid(z); the
    per-token MoE output sums w_e * y_e over the selected experts in ascending expert index.
R9  Activations are kept in the working precision (float32 by default) throughout; only the KV
    cache is stored in bf16. logits are float32.
R10 Greedy decoding takes the first index of the maximum logit.

Storage conventions (they are the boundary's layouts too)
--------------------------------------------------------
bf16 tensors are uint16 bit patterns (FP8 matrices: uint8 packed rows of K codes + 16 scale bytes,
see ``oracle.fp8``). embed/lm_head [V, H]; norms [H]; w_qkv [(Hq+2Hkv)*D, H]
with rows ordered q heads, then k heads, then v heads; w_o [H, Hq*D]; w_router [E, H];
w_gate/w_up [E, F, H]; w_down [E, H, F]; KV cache per layer [num_pages, Hkv, page, D] for K and
for V separately; block_tables [B, max_pages] int32 (page ids, -1 where unused).
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16, f64_to_bf16
from .fp8 import dequant_rows
from .mxfp4 import Mxfp4Rows, dequant_rows as mx_dequant_rows


@dataclass(frozen=True)
class Dims:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_ffn: int
    vocab: int
    page_size: int = 16
    rope_theta: float = 1e4
    rms_eps: float = 1e-6

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass
class LayerWeights:
    attn_norm: np.ndarray          # uint16 [H]
    w_qkv: np.ndarray              # uint16 [(Hq+2Hkv)D, H]
    w_o: np.ndarray                # uint16 [H, Hq D]
    w_router: np.ndarray           # uint16 [E, H]
    router_bias: Optional[np.ndarray]  # float32 [E] or None
    w_gate: np.ndarray             # uint16 [E, F, H]
    w_up: np.ndarray               # uint16 [E, F, H]
    w_down: np.ndarray             # uint16 [E, H, F]


@dataclass
class DenseWeights:
    """All weights held as host arrays. Other providers may duck-type ``embed_row``,
    ``layer(l)``, ``expert(l, e)``, ``final_norm`` and ``lm_head_rows``."""
    embed: np.ndarray              # uint16 [V, H]
    lm_head: np.ndarray            # uint16 [V, H]
    final_norm: np.ndarray         # uint16 [H]
    layers: list = field(default_factory=list)

    def embed_row(self, token):
        return self.embed[token]

    def layer(self, l):
        return self.layers[l]

    def expert(self, l, e):
        lw = self.layers[l]
        return lw.w_gate[e], lw.w_up[e], lw.w_down[e]

    def lm_head_rows(self, start, stop):
        return self.lm_head[start:stop]


@dataclass
class PagedKV:
    """Per-layer paged K and V caches (uint16 bf16 patterns) [num_pages, Hkv, page, D]."""
    k: list
    v: list


@dataclass
class StepResult:
    logits: Optional[np.ndarray]    # float32 [B, V] (None when the model has no lm_head)
    x_final: np.ndarray             # [B, H] residual stream after the last layer
    n_final: np.ndarray             # [B, H] final-normed hidden state (lm_head input)
    topk: np.ndarray                # int32 [L, B, k] selected experts, ascending index
    topk_weight: np.ndarray         # [L, B, k] router weights aligned with ``topk``
    router_logits: np.ndarray       # [L, B, E]
    margin: np.ndarray              # [L, B] r_(k) - r_(k+1) of the sorted logits (inf if k == E)
    x_layers: list                  # x_l for l = 0..L (x_0 = embedding)


# ----------------------------------------------------------------------------------------------
# pieces
# ----------------------------------------------------------------------------------------------

def _dec(a, dtype):
    """A stored tensor as values in ``dtype``: bf16 bit patterns (uint16), a matrix of packed MXFP4
    rows (``oracle.mxfp4.Mxfp4Rows``) or of packed FP8 rows (other uint8: E4M3 codes and a float32
    scale per row, ``oracle.fp8``), dequantized."""
    if isinstance(a, Mxfp4Rows):
        return mx_dequant_rows(a, dtype)
    if a.dtype == np.uint8:
        return dequant_rows(a, dtype)
    return bf16_to_f32(a).astype(dtype, copy=False)


def rmsnorm(x, gain, eps, dtype=np.float32):
    """R1: x / sqrt(mean(x^2) + eps) * gain, in ``dtype``."""
    x = np.asarray(x, dtype=dtype)
    ms = np.mean(x * x, dtype=dtype)
    return (x / np.sqrt(ms + dtype(eps))) * gain.astype(dtype, copy=False)


def rope_cos_sin(pos, head_dim, theta, dtype=np.float32):
    """R3: cos/sin of pos * theta^(-2i/D) for i < D/2; angle in float64, then cast to dtype."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.float64(pos) * inv_freq
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x, pos, theta, dtype=np.float32):
    """R3: rotate-half RoPE of the last axis of ``x`` (length D) at position ``pos``."""
    x = np.asarray(x, dtype=dtype)
    d = x.shape[-1]
    c, s = rope_cos_sin(pos, d, theta, dtype)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gather_paged(cache, block_table, n, page_size):
    """Keys/values 0..n-1 of one sequence from a paged cache [pages, Hkv, page, D] -> [n, Hkv, D]
    (P1 "From demo to a full serving system": paged attention)."""
    n_pages = (n + page_size - 1) // page_size
    ids = np.asarray(block_table[:n_pages], dtype=np.int64)
    blocks = cache[ids]                                  # [n_pages, Hkv, page, D]
    seq = np.transpose(blocks, (0, 2, 1, 3)).reshape(n_pages * page_size, cache.shape[1], cache.shape[3])
    return seq[:n]


def decode_attention(q, k, v, dtype=np.float32):
    """Single-query GQA attention (R4, R5). q [Hq, D]; k, v [n, Hkv, D] (already decoded).

    out[h] = softmax(k[:, g] @ q[h] / sqrt(D)) @ v[:, g] with g = h // (Hq / Hkv); the softmax
    subtracts the maximum score before exponentiating."""
    hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    scale = np.sqrt(dtype(d))
    out = np.empty((hq, d), dtype=dtype)
    for h in range(hq):
        g = h // grp
        s = (k[:, g, :] @ q[h]) / scale
        p = np.exp(s - np.max(s))
        out[h] = (p @ v[:, g, :]) / np.sum(p, dtype=dtype)
    return out


def route(r, top_k):
    """R7: indices of the top_k largest logits (ties -> lower index), returned in ascending index
    order, with their softmax-renormalised weights and the k-th/(k+1)-th margin."""
    r = np.asarray(r)
    order = np.argsort(-r, kind="stable")
    sel = order[:top_k]
    margin = (r[order[top_k - 1]] - r[order[top_k]]) if top_k < r.shape[0] else np.inf
    sel_sorted = np.sort(sel)
    rs = r[sel_sorted]
    e = np.exp(rs - np.max(rs))
    w = e / np.sum(e, dtype=r.dtype)
    return sel_sorted.astype(np.int32), w, margin


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (z.dtype.type(1) + np.exp(-z))


def expert_ffn(n, w_gate, w_up, w_down, dtype=np.float32):
    """R8 for one expert: W_down (SiLU(W_gate n) * (W_up n))."""
    g = _dec(w_gate, dtype) @ n
    u = _dec(w_up, dtype) @ n
    return _dec(w_down, dtype) @ (silu(g) * u)


# ----------------------------------------------------------------------------------------------
# the step
# ----------------------------------------------------------------------------------------------

def decode_step(dims, w, kv, tokens, positions, block_tables, seq_lens, dtype=np.float32,
                forced_topk=None, lm_head_chunk=8192):
    """One decode step for a batch (P1 "One persistent kernel for the whole decode step").

    Mutates ``kv``: the new K/V of every sequence is written at its position (R6).
    ``forced_topk`` maps (layer, b) -> expert ids to use instead of the oracle's own choice; the
    comparison harness uses it to replay a near-tied routing decision the GPU took differently.
    Tokens are processed one at a time, so rows of a batch never mix.
    """
    L, H, D = dims.n_layers, dims.hidden, dims.head_dim
    hq, hkv = dims.n_q_heads, dims.n_kv_heads
    B = len(tokens)
    enc = f32_to_bf16 if dtype == np.float32 else f64_to_bf16
    topk = np.zeros((L, B, dims.top_k), np.int32)
    topw = np.zeros((L, B, dims.top_k), dtype)
    rlog = np.zeros((L, B, dims.n_experts), dtype)
    margin = np.zeros((L, B), np.float64)

    x = np.stack([_dec(w.embed_row(int(t)), dtype) for t in tokens])  # [B, H]
    x_layers = [x.copy()]
    for l in range(L):
        lw = w.layer(l)
        wqkv = _dec(lw.w_qkv, dtype)
        wo = _dec(lw.w_o, dtype)
        wr = _dec(lw.w_router, dtype)
        x_next = np.empty_like(x)
        for b in range(B):
            pos, n_ctx = int(positions[b]), int(seq_lens[b])
            assert pos == n_ctx - 1, "positions[b] must equal seq_lens[b] - 1 (R6)"
            n = rmsnorm(x[b], _dec(lw.attn_norm, dtype), dims.rms_eps, dtype)
            # attention branch
            qkv = wqkv @ n
            q = qkv[: hq * D].reshape(hq, D)
            k_new = qkv[hq * D: (hq + hkv) * D].reshape(hkv, D)
            v_new = qkv[(hq + hkv) * D:].reshape(hkv, D)
            q = rope(q, pos, dims.rope_theta, dtype)
            k_new = rope(k_new, pos, dims.rope_theta, dtype)
            page = int(block_tables[b][pos // dims.page_size])
            slot = pos % dims.page_size
            kv.k[l][page, :, slot, :] = enc(k_new)
            kv.v[l][page, :, slot, :] = enc(v_new)
            kk = _dec(gather_paged(kv.k[l], block_tables[b], n_ctx, dims.page_size), dtype)
            vv = _dec(gather_paged(kv.v[l], block_tables[b], n_ctx, dims.page_size), dtype)
            attn = wo @ decode_attention(q, kk, vv, dtype).reshape(hq * D)
            # MoE branch, from the same normed input (R2)
            r = wr @ n
            if lw.router_bias is not None:
                r = r + lw.router_bias.astype(dtype)
            sel, wsel, mg = route(r, dims.top_k)
            if forced_topk is not None and (l, b) in forced_topk:
                sel = np.sort(np.asarray(forced_topk[(l, b)], dtype=np.int32))
                rs = r[sel]
                e = np.exp(rs - np.max(rs))
                wsel = e / np.sum(e, dtype=dtype)
            moe = np.zeros(H, dtype)
            for e_id, we in zip(sel, wsel):
                g_, u_, d_ = w.expert(l, int(e_id))
                moe += we * expert_ffn(n, g_, u_, d_, dtype)
            topk[l, b], topw[l, b], rlog[l, b], margin[l, b] = sel, wsel, r, mg
            x_next[b] = (x[b] + attn) + moe
        x = x_next
        x_layers.append(x.copy())

    gf = _dec(w.final_norm, dtype)
    n_final = np.stack([rmsnorm(x[b], gf, dims.rms_eps, dtype) for b in range(B)])
    logits = None
    if dims.vocab > 0:
        logits = np.empty((B, dims.vocab), np.float32)
        for s in range(0, dims.vocab, lm_head_chunk):
            e = min(dims.vocab, s + lm_head_chunk)
            wl = _dec(w.lm_head_rows(s, e), dtype)
            for b in range(B):
                logits[b, s:e] = (wl @ n_final[b]).astype(np.float32)
    return StepResult(logits, x, n_final, topk, topw, rlog, margin, x_layers)


def greedy_decode(dims, w, kv, tokens, positions, block_tables, seq_lens, steps, dtype=np.float32):
    """Free-running greedy decoding (R10): each step's argmax is the next step's token."""
    tokens = np.array(tokens, np.int64)
    positions = np.array(positions, np.int64)
    seq_lens = np.array(seq_lens, np.int64)
    out = []
    for _ in range(steps):
        res = decode_step(dims, w, kv, tokens, positions, block_tables, seq_lens, dtype)
        out.append(res)
        tokens = np.argmax(res.logits, axis=1)
        positions = positions + 1
        seq_lens = seq_lens + 1
    return out
