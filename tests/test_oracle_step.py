"""Pins of the oracle's whole decode step: structure and invariants that a wiring mistake
(wrong input to a branch, missing residual, K/V written late or at the wrong slot, rows mixing
across the batch, wrong precision handling) would break."""

import copy

import numpy as np
import pytest

import oracle
from oracle import bf16_to_f32, f32_to_bf16
from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.fixture(scope="module")
def tiny():
    s = harness.tiny_setup()
    s["dims"] = harness.dims_of(s["wl"])
    s["dw"] = harness.dense_weights(s["w"])
    s["kv"] = harness.host_kv(s["k"], s["v"])
    return s


def _step(s, kv=None, dtype=np.float32, dw=None, tokens=None, ctx=None, bt=None):
    kv = copy.deepcopy(s["kv"]) if kv is None else kv
    ctx = s["ctx"] if ctx is None else ctx
    toks = s["tokens"] if tokens is None else tokens
    return oracle.decode_step(s["dims"], dw or s["dw"], kv, toks, ctx.copy(),
                              s["block_tables"] if bt is None else bt, ctx + 1, dtype), kv


def test_fp32_matches_fp64(tiny):
    """The fp32 step agrees with the same definition evaluated in fp64 (R9's precision budget)."""
    r32, _ = _step(tiny)
    r64, _ = _step(tiny, dtype=np.float64)
    assert np.max(np.abs(r32.logits - r64.logits)) < 1e-4
    assert np.array_equal(r32.topk, r64.topk)


def test_kv_written_at_position_before_attention(tiny):
    """Slot pos of the sequence's page holds bf16(RoPE(k_new)) and bf16(v_new) after the step."""
    s = tiny
    r, kv = _step(s)
    d = s["dims"]
    pos = int(s["ctx"][0])
    page = s["block_tables"][0][pos // d.page_size]
    lw = s["dw"].layers[0]
    n = oracle.rmsnorm(bf16_to_f32(s["dw"].embed[s["tokens"][0]]), bf16_to_f32(lw.attn_norm), d.rms_eps)
    qkv = bf16_to_f32(lw.w_qkv) @ n
    hq, hkv, D = d.n_q_heads, d.n_kv_heads, d.head_dim
    k_new = oracle.rope(qkv[hq * D:(hq + hkv) * D].reshape(hkv, D), pos, d.rope_theta)
    v_new = qkv[(hq + hkv) * D:].reshape(hkv, D)
    assert np.array_equal(kv.k[0][page, :, pos % d.page_size], f32_to_bf16(k_new))
    assert np.array_equal(kv.v[0][page, :, pos % d.page_size], f32_to_bf16(v_new))
    # every other slot is untouched
    mask = np.ones(kv.k[0].shape[:3], bool)
    mask[page, :, pos % d.page_size] = False
    assert np.array_equal(kv.k[0][mask], s["kv"].k[0][mask])


def test_zero_branches_leave_residual_unchanged(tiny):
    """With W_o = 0 and W_down = 0 both branches add exactly zero: x_L == embedding."""
    dw = copy.deepcopy(tiny["dw"])
    for lw in dw.layers:
        lw.w_o[:] = 0
        lw.w_down[:] = 0
    r, _ = _step(tiny, dw=dw)
    assert np.array_equal(r.x_final[0], bf16_to_f32(dw.embed[tiny["tokens"][0]]))


def test_branches_share_the_normed_input(tiny):
    """Parallel layer: with MoE zeroed, layer 0 adds exactly W_o attention(n) where both the
    queries and the new key come from the same n the router sees."""
    s = tiny
    dw = copy.deepcopy(s["dw"])
    for lw in dw.layers:
        lw.w_down[:] = 0
    r, kv = _step(s, dw=dw)
    d = s["dims"]
    lw = dw.layers[0]
    pos = int(s["ctx"][0])
    x0 = bf16_to_f32(dw.embed[s["tokens"][0]])
    n = oracle.rmsnorm(x0, bf16_to_f32(lw.attn_norm), d.rms_eps)
    qkv = bf16_to_f32(lw.w_qkv) @ n
    D, hq = d.head_dim, d.n_q_heads
    q = oracle.rope(qkv[:hq * D].reshape(hq, D), pos, d.rope_theta)
    kk = bf16_to_f32(oracle.gather_paged(kv.k[0], s["block_tables"][0], pos + 1, d.page_size))
    vv = bf16_to_f32(oracle.gather_paged(kv.v[0], s["block_tables"][0], pos + 1, d.page_size))
    attn = bf16_to_f32(lw.w_o) @ oracle.decode_attention(q, kk, vv).reshape(-1)
    assert np.allclose(r.x_layers[1][0], x0 + attn, rtol=0, atol=1e-6)
    # the router saw the same n
    assert np.allclose(r.router_logits[0, 0], bf16_to_f32(lw.w_router) @ n, rtol=0, atol=1e-6)


def test_new_key_attends_to_itself(tiny):
    """A query aligned with the new key at a huge scale returns (almost) the new value: the new
    key is in the attended range and was written before attending."""
    s = tiny
    dw = copy.deepcopy(s["dw"])
    d = s["dims"]
    D, hq, hkv = d.head_dim, d.n_q_heads, d.n_kv_heads
    lw = dw.layers[0]
    # make q of head 0 and k of group 0 (dim 0 only) both a large multiple of n itself
    x0 = bf16_to_f32(dw.embed[s["tokens"][0]])
    n0 = oracle.rmsnorm(x0, bf16_to_f32(lw.attn_norm), d.rms_eps)
    row = f32_to_bf16((0.05 * n0).astype(np.float32))
    for t in range(D):
        lw.w_qkv[t] = row if t == 0 else 0                   # q head 0: only dim 0
        lw.w_qkv[hq * D + t] = row if t == 0 else 0          # k group 0: only dim 0
    r, kv = _step(s, dw=dw)
    pos = int(s["ctx"][0])
    x0 = bf16_to_f32(dw.embed[s["tokens"][0]])
    n = oracle.rmsnorm(x0, bf16_to_f32(lw.attn_norm), d.rms_eps)
    v_new = (bf16_to_f32(lw.w_qkv) @ n)[(hq + hkv) * D:(hq + hkv + 1) * D]
    q = oracle.rope((bf16_to_f32(lw.w_qkv) @ n)[:hq * D].reshape(hq, D), pos, d.rope_theta)
    kk = bf16_to_f32(oracle.gather_paged(kv.k[0], s["block_tables"][0], pos + 1, d.page_size))
    vv = bf16_to_f32(oracle.gather_paged(kv.v[0], s["block_tables"][0], pos + 1, d.page_size))
    out = oracle.decode_attention(q, kk, vv)
    scores = kk[:, 0, :] @ q[0] / np.sqrt(D)
    assert np.argmax(scores) == pos                           # the new key wins ...
    assert np.allclose(out[0], bf16_to_f32(f32_to_bf16(v_new)), atol=1e-3)  # ... and its value comes back


def test_batch_rows_are_independent():
    """Row b of a batch-2 step is bit-identical to a batch-1 step of sequence b alone."""
    wl = synth.workload("tiny", batch=2)
    s = harness.tiny_setup(wl)
    dims = harness.dims_of(wl)
    dw = harness.dense_weights(s["w"])
    kv = harness.host_kv(s["k"], s["v"])
    ctx = s["ctx"]
    r2 = oracle.decode_step(dims, dw, copy.deepcopy(kv), s["tokens"], ctx.copy(), s["block_tables"], ctx + 1)
    for b in range(2):
        r1 = oracle.decode_step(dims, dw, copy.deepcopy(kv), s["tokens"][b:b + 1], ctx[b:b + 1].copy(),
                                s["block_tables"][b:b + 1], ctx[b:b + 1] + 1)
        assert np.array_equal(r1.logits[0], r2.logits[b])
        assert np.array_equal(r1.topk[:, 0], r2.topk[:, b])


def test_greedy_tiny_runs_and_is_deterministic(tiny):
    """16 free-running greedy steps of the tiny model finish in seconds and repeat exactly."""
    s = tiny
    outs = []
    for _ in range(2):
        kv = copy.deepcopy(s["kv"])
        res = oracle.greedy_decode(s["dims"], s["dw"], kv, s["tokens"], s["ctx"], s["block_tables"],
                                   s["ctx"] + 1, 16)
        outs.append(np.array([np.argmax(r.logits, 1) for r in res]))
    assert outs[0].shape == (16, 1)
    assert np.array_equal(outs[0], outs[1])


def test_uniform_gains_change_the_result(tiny):
    """Gains are really applied (U(0.5,1.5) gains change the logits)."""
    s = harness.tiny_setup(gains="uniform")
    dims = harness.dims_of(s["wl"])
    r1 = oracle.decode_step(dims, harness.dense_weights(s["w"]), harness.host_kv(s["k"], s["v"]),
                            s["tokens"], s["ctx"].copy(), s["block_tables"], s["ctx"] + 1)
    r0, _ = _step(tiny)
    assert not np.allclose(r0.logits, r1.logits)
