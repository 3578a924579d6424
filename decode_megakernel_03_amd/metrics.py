"""Speed-of-light accounting for a decode step (host-side, no GPU work).

Decode is bound by HBM traffic: each step must stream the weights it touches plus the KV cache
it attends over, so the speed of light is peak bandwidth / bytes per step, and an engine's
efficiency is its achieved rate over that ceiling (P1 lede and "Decode is a bandwidth game").

For the MoE model the bytes a step *must* move are: every dense weight (QKV, O, router, norms),
the union over the batch of the routed experts' gate/up/down matrices (an expert touched by two
tokens of the batch is still read once), the lm_head, one embedding row per token, and the K and
V of every attended position. Partials, descriptors, counters and the 1-token KV write are
overheads, not part of the speed-of-light figure.
"""

import numpy as np

BF16 = 2


def matrix_bytes(wl, rows, k):
    """Stored bytes of a matrix of ``rows`` rows of ``k`` inputs: bf16; FP8 rows of k codes plus a
    16-byte tail holding the row's scale; or MXFP4 rows of k/2 code bytes and k/32 scale bytes padded
    to 16 bytes."""
    fmt = getattr(wl, "weights", "bf16")
    if fmt == "fp8":
        return rows * (k + 16)
    if fmt == "mxfp4":
        return rows * ((k // 2 + k // 32 + 15) // 16 * 16)
    return rows * k * BF16


def weight_bytes(wl, union_per_layer):
    """Weight bytes a step must read. ``union_per_layer``: distinct experts per layer (len L)."""
    H, D, F = wl.hidden, wl.head_dim, wl.expert_ffn
    dense = (matrix_bytes(wl, wl.qkv_rows, H) + matrix_bytes(wl, H, wl.n_q_heads * D)
             + matrix_bytes(wl, wl.n_experts, H) + H * BF16)
    expert = 2 * matrix_bytes(wl, F, H) + matrix_bytes(wl, H, F)
    lm = matrix_bytes(wl, wl.vocab, H) + H * BF16 if wl.lm_head else 0
    embed = wl.batch * H * BF16
    return int(wl.n_layers * dense + expert * int(np.sum(union_per_layer)) + lm + embed)


def kv_bytes(wl, seq_lens):
    """K and V bytes read by attention: every position of every sequence, every layer."""
    per_pos = 2 * wl.n_kv_heads * wl.head_dim * BF16
    return int(wl.n_layers * per_pos * int(np.sum(seq_lens)))


def step_bytes(wl, union_per_layer, seq_lens):
    return weight_bytes(wl, union_per_layer) + kv_bytes(wl, seq_lens)


def sol_tok_s(bytes_per_step, batch, peak_bytes_per_s):
    """Tokens/s if the step ran at peak bandwidth."""
    return batch * peak_bytes_per_s / bytes_per_step


def sol_fraction(tok_s, bytes_per_step, batch, peak_bytes_per_s):
    return tok_s / sol_tok_s(bytes_per_step, batch, peak_bytes_per_s)
