"""Pins of the speed-of-light accounting: the pages' own arithmetic (golden fixture) and the
byte count of a step, recomputed element by element from the shapes."""

import math
import os

import numpy as np

from decode_megakernel_03_amd import metrics, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sol_pages.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_sol_matches_pages():
    g = _golden()
    b = g["weight_bytes_per_step"] + g["kv_bytes_per_step"]
    sol = metrics.sol_tok_s(b, 1, g["hbm_bytes_per_s"])
    assert abs(sol - g["sol_tok_s_approx"]) < 5                         # "about 470"
    assert round(100 * metrics.sol_fraction(g["megakernel_tok_s"], b, 1, g["hbm_bytes_per_s"])) == g["megakernel_sol_pct"]
    assert round(100 * metrics.sol_fraction(g["vllm_tok_s"], b, 1, g["hbm_bytes_per_s"])) == g["vllm_sol_pct"]
    assert round(g["megakernel_tok_s"] / g["vllm_tok_s"], 2) == g["speedup"]


def test_step_bytes_by_enumeration():
    """Count every tensor of the full model one by one (bs1, 8K context, 8 experts per layer)."""
    wl = synth.workload("full")
    H, L = 2048, 48
    per_layer = {
        "qkv": (32 + 2 * 4) * 128 * H, "o": H * 32 * 128, "router": 128 * H, "norm": H,
        "experts": 8 * (768 * H + 768 * H + H * 768),
    }
    total = L * sum(per_layer.values()) * 2 + (151936 * H + H) * 2 + H * 2
    kv = L * 8192 * (2 * 4 * 128 * 2)
    assert metrics.step_bytes(wl, np.full(L, 8), [8192]) == total + kv
    # 6.08 GB of weights and 0.81 GB of KV, as the shapes imply
    assert math.isclose(total / 1e9, 6.0835, abs_tol=1e-3) and math.isclose(kv / 1e9, 0.8053, abs_tol=1e-3)

