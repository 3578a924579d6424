"""Pins of the oracle's pieces against things other than the oracle itself: closed forms,
hand-computed values, invariants, brute force and independent library routines.

Each test says which mistake it would catch."""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import (bf16_to_f32, f32_to_bf16, f64_to_bf16, rmsnorm, rope, rope_cos_sin,
                    decode_attention, gather_paged, route, silu, expert_ffn)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- bf16 codec

def test_bf16_roundtrip_exhaustive():
    """Every one of the 65536 patterns decodes exactly and re-encodes to itself (NaN stays NaN)."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(pats)
    back = f32_to_bf16(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], pats[~nan])
    assert np.all(np.isnan(bf16_to_f32(back[nan])))
    # the decoded float's top half is the pattern and the bottom half is zero
    assert np.all((f.view(np.uint32) & 0xFFFF) == 0)


def test_bf16_encode_matches_torch():
    """Round-to-nearest-even against torch's float32 -> bfloat16 conversion (independent code):
    random values, exact ties between neighbours, near-ties, overflow to inf, subnormals."""
    rng = np.random.default_rng(0)
    vals = [rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000)]
    base = rng.integers(0, 2 ** 16, 20000).astype(np.uint32) << 16
    for off in (0x8000, 0x7FFF, 0x8001, 0x0001, 0xFFFF):       # exact tie, just below, just above ...
        vals.append((base | off).view(np.float32))
    vals.append(np.array([3.3895314e38, 3.4028235e38, -3.4e38, 1e-40, -1e-41, 0.0, -0.0, np.inf, -np.inf], np.float32))
    x = np.concatenate(vals).astype(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16(x), ref)


def test_bf16_ties_to_even_by_hand():
    # 1 + 2^-8 is halfway between 1 (even mantissa) and 1 + 2^-7 -> rounds to 1.0 (0x3F80)
    assert f32_to_bf16(np.float32(1 + 2 ** -8)) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> rounds up to 0x3F82
    assert f32_to_bf16(np.float32(1 + 3 * 2 ** -8)) == 0x3F82
    assert f32_to_bf16(np.float32(-2.0)) == 0xC000


def test_f64_to_bf16_is_nearest():
    """Direct fp64 rounding picks the nearest bf16 (ties to even) - brute force over neighbours."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * 10.0 ** rng.integers(-5, 5, 20000)
    got = f64_to_bf16(x)
    # candidates: the truncation of the float32 rounding and its neighbours
    t = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    cands = np.stack([t - 1, t, t + 1], 1)
    cv = bf16_to_f32((cands & 0xFFFF).astype(np.uint16)).astype(np.float64)
    err = np.abs(cv - x[:, None])
    best = cands[np.arange(len(x)), np.argmin(err, 1)]
    gv = bf16_to_f32(got).astype(np.float64)
    assert np.all(np.abs(gv - x) <= err.min(1))          # nearest
    exact_tie = np.sum(err == err.min(1, keepdims=True), 1) > 1
    assert np.array_equal(got[~exact_tie], (best[~exact_tie] & 0xFFFF).astype(np.uint16))


# ---------------------------------------------------------------- GEMV (matmul as a step)

def test_gemv_within_fp32_dot_bound():
    """The oracle's fp32 matrix-vector products stay within the textbook bound
    |fl(a.b) - a.b| <= gamma_n * sum|a_i b_i|, gamma_n = n u / (1 - n u), u = 2^-24."""
    rng = np.random.default_rng(2)
    n = 2048
    W = bf16_to_f32(f32_to_bf16((rng.standard_normal((512, n)) * 0.02).astype(np.float32)))
    x = rng.standard_normal(n).astype(np.float32)
    y32 = W @ x
    y64 = W.astype(np.float64) @ x.astype(np.float64)
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64)))
    assert np.all(np.abs(y32 - y64) <= bound)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_value():
    # x = (3, 4): mean square 12.5; n = x / sqrt(12.5 + eps)
    g = f32_to_bf16(np.ones(2, np.float32))
    n = rmsnorm(np.array([3.0, 4.0]), bf16_to_f32(g), 1e-6, np.float64)
    assert np.allclose(n, [3 / math.sqrt(12.5 + 1e-6), 4 / math.sqrt(12.5 + 1e-6)], rtol=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(2048)
    g = bf16_to_f32(f32_to_bf16(rng.uniform(0.5, 1.5, 2048).astype(np.float32)))
    ones = np.ones(2048, np.float32)
    n1 = rmsnorm(x, ones, 1e-6, np.float64)
    ms = np.mean(x * x)
    # output RMS is sqrt(ms / (ms + eps)) with unit gain
    assert math.isclose(math.sqrt(np.mean(n1 * n1)), math.sqrt(ms / (ms + 1e-6)), rel_tol=1e-12)
    # scaling x by c only changes how much eps weighs: n(cx) = n(x) sqrt((ms + eps) / (ms + eps / c^2))
    c = 1000.0
    assert np.allclose(rmsnorm(c * x, ones, 1e-6, np.float64), n1 * math.sqrt((ms + 1e-6) / (ms + 1e-6 / c ** 2)), rtol=1e-12)
    # the gain multiplies elementwise after normalising
    assert np.allclose(rmsnorm(x, g, 1e-6, np.float64), n1 * g, rtol=1e-14)
    # eps matters: a zero vector maps to zero, not NaN
    assert np.all(rmsnorm(np.zeros(8), np.ones(8, np.float32), 1e-6, np.float64) == 0)


# ---------------------------------------------------------------- RoPE

def test_rope_inv_freq_values():
    # theta^(-2i/D) at D=128, theta=1e4: i=0 -> 1, i=32 -> 1e4^-0.5 = 0.01, i=16 -> 1e4^-0.25 = 0.1
    c, s = rope_cos_sin(1, 128, 1e4, np.float64)
    assert math.isclose(math.atan2(s[0], c[0]), 1.0, rel_tol=1e-14)
    assert math.isclose(math.atan2(s[32], c[32]), 0.01, rel_tol=1e-12)
    assert math.isclose(math.atan2(s[16], c[16]), 0.1, rel_tol=1e-12)


def test_rope_vs_complex_multiply():
    """Rotate-half RoPE equals multiplying z_i = x_i + 1j*x_{i+D/2} by exp(1j*pos*theta^(-2i/D))."""
    rng = np.random.default_rng(4)
    for D, pos in [(32, 0), (32, 77), (128, 8192), (128, 262143)]:
        x = rng.standard_normal((5, D))
        got = rope(x, pos, 1e4, np.float64)
        z = x[:, : D // 2] + 1j * x[:, D // 2:]
        ang = pos * 1e4 ** (-2.0 * np.arange(D // 2) / D)
        zr = z * np.exp(1j * ang)
        ref = np.concatenate([zr.real, zr.imag], axis=1)
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    assert np.array_equal(rope(q, 0, 1e4, np.float64), q)                     # pos 0 = identity
    r = rope(q, 1234, 1e4, np.float64)
    assert np.allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2)   # per-pair norm
    # the score depends only on the relative offset p - p'
    a = rope(q, 100, 1e4, np.float64) @ rope(k, 40, 1e4, np.float64)
    b = rope(q, 1060, 1e4, np.float64) @ rope(k, 1000, 1e4, np.float64)
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_fp32_angle_formed_in_fp64():
    """At large positions the fp32 cos/sin must come from an fp64 angle: compare with the
    correctly rounded value computed at higher precision via math.fsum-free python floats."""
    c, s = rope_cos_sin(262143, 128, 1e4, np.float32)
    for i in (0, 1, 5, 63):
        ang = 262143 * (1e4 ** (-2.0 * i / 128))
        assert c[i] == np.float32(math.cos(ang)) and s[i] == np.float32(math.sin(ang))


# ---------------------------------------------------------------- attention

def _attention_loops(q, k, v):
    """Explicit per-head, per-key loops in float64."""
    hq, d = q.shape
    n, hkv, _ = k.shape
    out = np.zeros((hq, d))
    for h in range(hq):
        g = h // (hq // hkv)
        scores = []
        for j in range(n):
            s = 0.0
            for t in range(d):
                s += q[h, t] * k[j, g, t]
            scores.append(s / math.sqrt(d))
        m = max(scores)
        p = [math.exp(s - m) for s in scores]
        tot = sum(p)
        for t in range(d):
            out[h, t] = sum(p[j] * v[j, g, t] for j in range(n)) / tot
    return out


@pytest.mark.parametrize("n", [1, 7, 33])
def test_attention_vs_loops(n):
    rng = np.random.default_rng(6 + n)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((n, 2, 8))
    v = rng.standard_normal((n, 2, 8))
    assert np.allclose(decode_attention(q, k, v, np.float64), _attention_loops(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 8))
    k1, v1 = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 8))
    out = decode_attention(q, k1, v1, np.float64)                    # one key -> its value
    assert np.allclose(out[:2], v1[0, 0]) and np.allclose(out[2:], v1[0, 1])
    k = np.repeat(rng.standard_normal((1, 2, 8)), 9, axis=0)         # identical keys -> mean(V)
    v = rng.standard_normal((9, 2, 8))
    out = decode_attention(q, k, v, np.float64)
    assert np.allclose(out[0], v[:, 0].mean(0)) and np.allclose(out[3], v[:, 1].mean(0))
    k = rng.standard_normal((9, 2, 8)) * 0.01                        # one dominant score -> its value
    k[4, 0] = q[0] * 1000
    out = decode_attention(q, k, v, np.float64)
    assert np.allclose(out[0], v[4, 0], atol=1e-9)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((8, 16))
    k = rng.standard_normal((20, 2, 16))
    v = rng.standard_normal((20, 2, 16))
    mha = decode_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), np.float64)
    assert np.allclose(decode_attention(q, k, v, np.float64), mha, rtol=1e-13)


def test_paged_gather_equals_contiguous():
    """A sequence scattered over shuffled pages is read back bit-identically."""
    rng = np.random.default_rng(9)
    n, hkv, d, page = 70, 2, 8, 16
    contig = rng.integers(0, 2 ** 16, (n, hkv, d)).astype(np.uint16)
    n_pages = (n + page - 1) // page
    table = rng.permutation(12)[:n_pages].astype(np.int32)
    cache = rng.integers(0, 2 ** 16, (12, hkv, page, d)).astype(np.uint16)
    for j in range(n):
        cache[table[j // page], :, j % page, :] = contig[j]
    assert np.array_equal(gather_paged(cache, np.concatenate([table, [-1, -1]]), n, page), contig)
    # page size 1 and "one page holding everything" give the same sequence
    c1 = contig[:, :, None, :]
    assert np.array_equal(gather_paged(c1, np.arange(n), n, 1), contig)


# ---------------------------------------------------------------- routing

def _topk_bruteforce(r, k):
    """Rank = number of logits that beat r_e (larger, or equal with a lower index)."""
    sel = []
    for e in range(len(r)):
        rank = sum(1 for f in range(len(r)) if r[f] > r[e] or (r[f] == r[e] and f < e))
        if rank < k:
            sel.append(e)
    return sel


def test_topk_vs_bruteforce_with_ties():
    rng = np.random.default_rng(10)
    for trial in range(300):
        E, k = [(8, 2), (128, 8), (16, 5)][trial % 3]
        r = rng.standard_normal(E).astype(np.float32)
        if trial % 2:                                   # force ties, also across the k boundary
            r = np.round(r * 2) / 2
        sel, w, margin = route(r, k)
        assert list(sel) == _topk_bruteforce(r, k)
        srt = np.sort(r)[::-1]
        assert margin == srt[k - 1] - srt[k]


def test_topk_all_equal_takes_lowest_indices():
    sel, w, _ = route(np.zeros(128, np.float32), 8)
    assert list(sel) == list(range(8))
    assert np.allclose(w, 1 / 8)


def test_router_weights_are_renormalised_softmax():
    rng = np.random.default_rng(11)
    r = rng.standard_normal(128)
    sel, w, _ = route(r, 8)
    full = np.exp(r - r.max()) / np.exp(r - r.max()).sum()
    assert math.isclose(w.sum(), 1.0, rel_tol=1e-14)
    assert np.allclose(w, full[sel] / full[sel].sum(), rtol=1e-13)
    # shifting every logit by a constant (a uniform bias) changes nothing
    sel2, w2, _ = route(r + 3.0, 8)
    assert np.array_equal(sel, sel2) and np.allclose(w, w2)


# ---------------------------------------------------------------- SiLU / experts

def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 50.0, -50.0, -1000.0])
    s = silu(z)
    assert s[0] == 0.0
    assert math.isclose(s[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(s[2], -1 / (1 + math.e), rel_tol=1e-15)
    assert math.isclose(s[3], 50.0, rel_tol=1e-15) and abs(s[4]) < 1e-19 and s[5] == 0.0


def test_moe_sparse_equals_dense_masked_loop():
    """Sum over the selected experts == dense loop over every expert with zero weight elsewhere."""
    rng = np.random.default_rng(12)
    E, F, H, k = 8, 16, 32, 3
    enc = lambda a: f32_to_bf16(a.astype(np.float32))
    wg, wu, wd = enc(rng.standard_normal((E, F, H)) * 0.2), enc(rng.standard_normal((E, F, H)) * 0.2), enc(rng.standard_normal((E, H, F)) * 0.2)
    n = rng.standard_normal(H)
    r = rng.standard_normal(E)
    sel, w, _ = route(r, k)
    sparse = sum(wi * expert_ffn(n, wg[e], wu[e], wd[e], np.float64) for e, wi in zip(sel, w))
    mask = np.zeros(E)
    mask[sel] = w
    dense = np.zeros(H)
    G, U, Dn = bf16_to_f32(wg).astype(np.float64), bf16_to_f32(wu).astype(np.float64), bf16_to_f32(wd).astype(np.float64)
    for e in range(E):
        for f in range(F):
            g = sum(G[e, f, t] * n[t] for t in range(H))
            u = sum(U[e, f, t] * n[t] for t in range(H))
            hval = g / (1 + math.exp(-g)) * u
            for o in range(H):
                dense[o] += mask[e] * Dn[e, o, f] * hval
    assert np.allclose(sparse, dense, rtol=1e-12, atol=1e-12)
