"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle harness.

This module holds no arithmetic of the decode step itself: it only draws weights, KV pages,
tokens, sequence lengths and block tables from fixed seeds. Both the HIP path and the CPU oracle
receive the arrays it returns (the oracle as uint16 bf16 patterns, the HIP path as device tensors).

Workloads (shapes follow the parallel-MoE decoders the method is benchmarked on, P1 lede and
"Decode is a bandwidth game": 30B total / ~3B active, 8K context, batch 1 and 8):

* ``tiny``    - 2 layers, hidden 256, 8 Q / 2 KV heads of 32, 8 experts top-2, FFN 128, vocab 1024,
                batch 1, 64 prefilled positions, 16 greedy steps.
* ``layer``   - one full-shape layer (hidden 2048, 32 Q / 4 KV heads of 128, 128 experts top-8,
                FFN 768), no lm_head, batch 1, 8192 prefilled positions, one step; the layer input
                is an embedding row drawn N(0, 1).
* ``full``    - 48 full-shape layers, vocab 151936 with an untied lm_head, batch 1, 8192 context.
* ``full_b8`` - the same model at batch 8, 8192 context each.
* ``ragged``  - the same model at batch 8 with contexts log-uniform in [1024, 32768], shuffled
                block tables and a Zipf(1.1) router bias.
* ``ragged_uniform`` - the ragged batch without the router bias (uniform-routing control).
* ``long``    - the same model at batch 1 with 262144 context.
* ``tiny_fp8``, ``full_fp8``, ``full_b8_fp8`` - ``tiny``, ``full`` and ``full_b8`` with FP8 matrices.
* ``tiny_mxfp4``, ``full_mxfp4``, ``full_b8_mxfp4`` - the same with MXFP4 matrices.

Distributions: weights N(0, 0.02) rounded to bf16 (FP8 workloads: each matrix row of those then
stored as OCP E4M3 codes with a float32 absmax scale, max |w| / 448, codes rounded to nearest even;
MXFP4 workloads: each block of 32 inputs of a row stored as E2M1 codes with a shared power-of-two
scale 2^(floor(log2 max |w|) - 2), codes rounded to nearest even and clamped to +-6);
norm gains 1.0 (or U(0.5, 1.5) when asked,
so that gain mistakes cannot hide); K/V N(0, 1) rounded to bf16; tokens uniform in [0, V).
Every tensor has its own generator seeded from (seed, tensor index).
"""

from dataclasses import dataclass, replace
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_ffn: int
    vocab: int
    batch: int
    context: int            # prefilled positions per sequence (fixed-length workloads)
    steps: int
    page_size: int = 16
    rope_theta: float = 1e4
    rms_eps: float = 1e-6
    ragged: tuple = ()      # (lo, hi) for log-uniform context lengths
    zipf_s: float = 0.0     # router bias exponent (0 = no bias)
    lm_head: bool = True    # False: the step ends at the residual stream (single-layer test)
    embed_std: float = 0.02 # the single-layer test feeds N(0, 1) rows as the layer input
    weights: str = "bf16"   # matrix storage: "bf16", "fp8" (E4M3 codes + float32 row scale) or
                            # "mxfp4" (E2M1 codes, an E8M0 scale per block of 32)

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


_FULL = dict(n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128, n_experts=128,
             top_k=8, expert_ffn=768, vocab=151936)

WORKLOADS = {
    "tiny": Workload("tiny", n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=32,
                     n_experts=8, top_k=2, expert_ffn=128, vocab=1024, batch=1, context=64, steps=16),
    "layer": Workload("layer", **{**_FULL, "n_layers": 1, "vocab": 1024}, batch=1, context=8192, steps=1,
                      lm_head=False, embed_std=1.0),
    "full": Workload("full", **_FULL, batch=1, context=8192, steps=1024),
    "full_b8": Workload("full_b8", **_FULL, batch=8, context=8192, steps=1024),
    "ragged": Workload("ragged", **_FULL, batch=8, context=0, steps=1024, ragged=(1024, 32768), zipf_s=1.1),
    # the uniform-routing control of the ragged batch (same contexts and pages, no router bias)
    "ragged_uniform": Workload("ragged_uniform", **_FULL, batch=8, context=0, steps=1024, ragged=(1024, 32768)),
    "long": Workload("long", **_FULL, batch=1, context=262144, steps=256),
    "tiny_fp8": Workload("tiny_fp8", n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=32,
                         n_experts=8, top_k=2, expert_ffn=128, vocab=1024, batch=1, context=64, steps=16,
                         weights="fp8"),
    "full_fp8": Workload("full_fp8", **_FULL, batch=1, context=8192, steps=1024, weights="fp8"),
    "full_b8_fp8": Workload("full_b8_fp8", **_FULL, batch=8, context=8192, steps=1024, weights="fp8"),
    "tiny_mxfp4": Workload("tiny_mxfp4", n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=32,
                           n_experts=8, top_k=2, expert_ffn=128, vocab=1024, batch=1, context=64, steps=16,
                           weights="mxfp4"),
    "full_mxfp4": Workload("full_mxfp4", **_FULL, batch=1, context=8192, steps=1024, weights="mxfp4"),
    "full_b8_mxfp4": Workload("full_b8_mxfp4", **_FULL, batch=8, context=8192, steps=1024, weights="mxfp4"),
}


def workload(name, **over):
    w = WORKLOADS[name]
    return replace(w, **over) if over else w


def _gen(seed, idx, device):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(idx) * 7919 + 12345) % (2 ** 63 - 1))
    return g


def normal_bf16(shape, std, seed, idx, device="cpu"):
    """N(0, std) drawn in float32, rounded to bf16 by torch (round to nearest even)."""
    g = _gen(seed, idx, device)
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    # draw in slabs along the first axis to bound the float32 temporary
    n0 = shape[0]
    per = max(1, (1 << 27) // max(1, int(np.prod(shape[1:])) if len(shape) > 1 else 1))
    for s in range(0, n0, per):
        e = min(n0, s + per)
        t[s:e] = (torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    return t


def uniform_bf16(shape, lo, hi, seed, idx, device="cpu"):
    g = _gen(seed, idx, device)
    return (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo).to(torch.bfloat16)


def zipf_router_bias(wl, seed=4):
    """Per-layer router bias ln p_{pi_l(e)} - mean, p_r ~ r^-s over ranks r = 1..E, pi_l a seeded
    permutation per layer (a skewed, 'real-like' expert load)."""
    rng = np.random.default_rng([seed, 77])
    ranks = np.arange(1, wl.n_experts + 1, dtype=np.float64)
    logp = -wl.zipf_s * np.log(ranks)
    logp -= np.log(np.sum(np.exp(logp)))
    out = []
    for _ in range(wl.n_layers):
        perm = rng.permutation(wl.n_experts)
        b = logp[perm]
        out.append((b - b.mean()).astype(np.float32))
    return out


FP8_MAX = 448.0          # largest finite OCP E4M3 value


def quantize_rows_fp8(t):
    """A bf16 matrix [..., K] as packed FP8 rows uint8 [..., K + 16]: scale s = max |row| / 448 (1 for a
    zero row), codes E4M3(row / s) rounded to nearest even, then the float32 scale and 12 zero bytes."""
    x = t.float()
    amax = x.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (x / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    del x
    tail = torch.zeros(codes.shape[:-1] + (16,), dtype=torch.uint8, device=codes.device)
    tail[..., :4] = scale.to(torch.float32).contiguous().view(torch.uint8)
    return torch.cat([codes, tail], dim=-1).contiguous()


# E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 are codes 0..7; a magnitude rounds to the code that counts
# the midpoints below it, a tie going to the even code (the midpoints 0.25, 1.25, 2.5 and 5 round
# down, 0.75, 1.75 and 3.5 up)
_E2M1_MID_DOWN = (0.25, 1.25, 2.5, 5.0)
_E2M1_MID_UP = (0.75, 1.75, 3.5)


def mxfp4_row_bytes(k):
    """Bytes of one packed MXFP4 row of ``k`` inputs: k/2 code bytes and k/32 scale bytes, padded to 16."""
    return (k // 2 + k // 32 + 15) // 16 * 16


def quantize_rows_mxfp4(t):
    """A bf16 matrix [..., K] (K a multiple of 32) as packed MXFP4 rows uint8 [..., mxfp4_row_bytes(K)]:
    per block of 32 inputs the E8M0 scale byte 127 + floor(log2 max |w|) - 2 (127 for a zero block),
    codes E2M1(w / scale) rounded to nearest even and clamped to 6; two codes per byte, the even
    element in the low nibble; then the K/32 scale bytes and zero bytes."""
    k = t.shape[-1]
    assert k % 32 == 0
    x = t.float().reshape(t.shape[:-1] + (k // 32, 32))
    amax = x.abs().amax(dim=-1, keepdim=True)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.zeros_like(amax)).clamp(-127, 127)
    a = (x * torch.exp2(-e)).reshape(t.shape)
    del x
    mag = a.abs()
    code = torch.zeros(mag.shape, dtype=torch.uint8, device=t.device)
    for m in _E2M1_MID_DOWN:
        code += (mag > m).to(torch.uint8)
    for m in _E2M1_MID_UP:
        code += (mag >= m).to(torch.uint8)
    code |= (a < 0).to(torch.uint8) << 3
    del a, mag
    out = torch.zeros(t.shape[:-1] + (mxfp4_row_bytes(k),), dtype=torch.uint8, device=t.device)
    out[..., : k // 2] = code[..., 0::2] | (code[..., 1::2] << 4)
    out[..., k // 2: k // 2 + k // 32] = (e[..., 0] + 127).to(torch.uint8)
    return out


def make_weights(wl, seed=0, device="cpu", gains="ones", router_bias=None):
    """All model weights as torch tensors on ``device`` (bf16 unless noted; with FP8 or MXFP4 weights
    every matrix is uint8 packed rows, ``quantize_rows_fp8`` / ``quantize_rows_mxfp4``). The dict's
    "format" names the matrix storage (the workload's ``weights``)."""
    mat = {"fp8": quantize_rows_fp8, "mxfp4": quantize_rows_mxfp4}.get(wl.weights, lambda t: t)
    H, V = wl.hidden, wl.vocab
    w = {"format": wl.weights}
    i = 0

    def nxt():
        nonlocal i
        i += 1
        return i

    def gain(idx):
        if gains == "ones":
            return torch.ones(H, dtype=torch.bfloat16, device=device)
        return uniform_bf16((H,), 0.5, 1.5, seed, idx, device)

    w["embed"] = normal_bf16((V, H), wl.embed_std, seed, nxt(), device)
    lm_idx = nxt()
    w["lm_head"] = mat(normal_bf16((V, H), 0.02, seed, lm_idx, device)) if wl.lm_head else None
    w["final_norm"] = gain(nxt())
    layers = []
    for l in range(wl.n_layers):
        lw = {
            "attn_norm": gain(nxt()),
            "w_qkv": mat(normal_bf16((wl.qkv_rows, H), 0.02, seed, nxt(), device)),
            "w_o": mat(normal_bf16((H, wl.n_q_heads * wl.head_dim), 0.02, seed, nxt(), device)),
            "w_router": mat(normal_bf16((wl.n_experts, H), 0.02, seed, nxt(), device)),
            "w_gate": mat(normal_bf16((wl.n_experts, wl.expert_ffn, H), 0.02, seed, nxt(), device)),
            "w_up": mat(normal_bf16((wl.n_experts, wl.expert_ffn, H), 0.02, seed, nxt(), device)),
            "w_down": mat(normal_bf16((wl.n_experts, H, wl.expert_ffn), 0.02, seed, nxt(), device)),
            "router_bias": None,
        }
        if router_bias is not None:
            lw["router_bias"] = torch.as_tensor(router_bias[l], dtype=torch.float32, device=device)
        layers.append(lw)
    w["layers"] = layers
    return w


def context_lengths(wl, seed=3):
    """Prefilled context per sequence: fixed, or log-uniform in wl.ragged."""
    if not wl.ragged:
        return np.full(wl.batch, wl.context, np.int64)
    rng = np.random.default_rng([seed, 11])
    lo, hi = wl.ragged
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=wl.batch))).astype(np.int64)


def make_block_tables(ctx, extra_steps, page_size, seed=1, shuffle=True, spare_pages=0):
    """Shuffled page assignment with room for ``extra_steps`` more tokens per sequence.

    Returns (block_tables int32 [B, max_pages] padded with -1, num_pages)."""
    ctx = np.asarray(ctx, np.int64)
    need = [int((c + extra_steps + page_size - 1) // page_size) for c in ctx]
    total = int(sum(need)) + spare_pages
    rng = np.random.default_rng([seed, 5])
    ids = rng.permutation(total) if shuffle else np.arange(total)
    max_pages = max(need)
    bt = np.full((len(ctx), max_pages), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = ids[o:o + n]
        o += n
    return bt, total


def make_kv(wl, num_pages, seed=1, device="cpu", n_layers=None):
    """Per-layer K and V caches [num_pages, Hkv, page, D], N(0,1) rounded to bf16 (read as
    already-rotated keys). Unused slots hold values too; they are never read."""
    L = wl.n_layers if n_layers is None else n_layers
    shape = (num_pages, wl.n_kv_heads, wl.page_size, wl.head_dim)
    k = [normal_bf16(shape, 1.0, seed, 1000 + 2 * l, device) for l in range(L)]
    v = [normal_bf16(shape, 1.0, seed, 1001 + 2 * l, device) for l in range(L)]
    return k, v


def refill_sequence(wl, k, v, bt, b, new_ctx, extra_steps, seed):
    """Continuous batching: sequence slot b has hit its length and restarts with a fresh prompt of
    new_ctx positions. Its pages are reshuffled (seeded) and the ones covering the new prompt get
    fresh N(0,1) K/V in every layer (in place, on whatever device k and v live). Returns the slot's
    new block-table row (the same pages, in the new order) and the new sequence's first token."""
    row = np.asarray(bt[b])
    pages = row[row >= 0]
    need = int((new_ctx + extra_steps + wl.page_size - 1) // wl.page_size)
    if need > len(pages):
        raise ValueError(f"slot {b} owns {len(pages)} pages, the new sequence needs {need}")
    rng = np.random.default_rng([seed, 13, b])
    pages = rng.permutation(pages)
    out = np.full(row.shape, -1, np.int32)
    out[:len(pages)] = pages
    shape = (need, wl.n_kv_heads, wl.page_size, wl.head_dim)
    for l in range(len(k)):
        idx = torch.as_tensor(pages[:need].astype(np.int64), device=k[l].device)
        k[l][idx] = normal_bf16(shape, 1.0, seed, 5000 + 2 * l, k[l].device)
        v[l][idx] = normal_bf16(shape, 1.0, seed, 5001 + 2 * l, v[l].device)
    token = int(rng.integers(0, max(wl.vocab, 1)))
    return out, token


def prefill_pages(wl, k, v, pages, prompt_len, seed):
    """Synthetic prefill of a new sequence: seeded N(0,1) bf16 K/V for positions [0, prompt_len) in the
    pages it owns (in position order), in every layer, in place on whatever device k and v live."""
    need = int((int(prompt_len) + wl.page_size - 1) // wl.page_size)
    if need > len(pages):
        raise ValueError(f"{len(pages)} pages cannot hold {prompt_len} positions")
    if need == 0:
        return
    shape = (need, wl.n_kv_heads, wl.page_size, wl.head_dim)
    for l in range(len(k)):
        idx = torch.as_tensor(np.asarray(pages[:need], np.int64), device=k[l].device)
        k[l][idx] = normal_bf16(shape, 1.0, seed, 7000 + 2 * l, k[l].device)
        v[l][idx] = normal_bf16(shape, 1.0, seed, 7001 + 2 * l, v[l].device)


def synthetic_requests(wl, seed, n, ctx=(1024, 32768), new_tokens=(1, 1024)):
    """n requests of the ragged workload's refill rule: prompt length log-uniform in ctx, output budget
    uniform in new_tokens (inclusive), first token uniform in [0, V). Returns (prompt_len, max_new, token)."""
    rng = np.random.default_rng([seed, 17])
    c = np.floor(np.exp(rng.uniform(math.log(ctx[0]), math.log(ctx[1]), size=n))).astype(np.int64)
    o = rng.integers(new_tokens[0], new_tokens[1] + 1, size=n)
    t = rng.integers(0, max(wl.vocab, 1), size=n)
    return [(int(c[i]), int(o[i]), int(t[i])) for i in range(n)]


def synthetic_prompts(wl, seed, n, ctx=(1, 64), new_tokens=(1, 8)):
    """n requests that carry their prompts: length log-uniform in ctx, tokens uniform in [0, V), output
    budget uniform in new_tokens (inclusive). Returns (prompt tokens, max_new)."""
    rng = np.random.default_rng([seed, 23])
    c = np.floor(np.exp(rng.uniform(math.log(ctx[0]), math.log(ctx[1] + 1), size=n))).astype(np.int64)
    c = np.clip(c, ctx[0], ctx[1])
    o = rng.integers(new_tokens[0], new_tokens[1] + 1, size=n)
    return [(rng.integers(0, max(wl.vocab, 1), size=int(c[i])).astype(np.int32), int(o[i])) for i in range(n)]


def first_tokens(wl, seed=2):
    rng = np.random.default_rng([seed, 3])
    return rng.integers(0, max(wl.vocab, 1), size=wl.batch).astype(np.int32)


def to_u16(t):
    """bf16 torch tensor (any device) -> numpy uint16 bit patterns on the host."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def to_host(t):
    """A stored tensor on the host as the oracle reads it: bf16 -> uint16 patterns; packed FP8 or
    MXFP4 rows (uint8) -> uint8."""
    if t.dtype == torch.uint8:
        return t.detach().to("cpu").contiguous().numpy()
    return to_u16(t)
