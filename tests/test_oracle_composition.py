"""Pins of how the oracle's decode step puts its pinned pieces together.

The pieces (RMSNorm, RoPE, attention, paging, top-k routing, renormalised router weights, the
expert FFN) are each pinned in test_oracle_pieces.py. These tests pin the wiring between them:

* the MoE branch: the experts read the layer's *normed* input, each selected expert's output is
  scaled by its softmax weight renormalised over the selected set, and the sum joins the residual
  (parallel layer, P1 "One persistent kernel for the whole decode step"; SiLU-multiply expert,
  P3 "Key Technologies and Architecture");
* the final RMSNorm (with its own gain) between the last layer and the lm_head;
* a forced routing decision (the near-tie replay) weighs the forced experts by the softmax of
  their logits renormalised over the forced set.

Each wiring check has a special case that needs no re-derivation (identical experts, one-hot
lm_head rows, exact scale invariance) and a composition of the pinned pieces; each also shows that
the plausible mistakes (experts fed x instead of n, unrenormalised or dropped weights, the final
norm or its gain skipped) land far outside the tolerance used.
"""

import copy
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import bf16_to_f32, f32_to_bf16
from tests import harness

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _setup(gains="uniform"):
    s = harness.tiny_setup(gains=gains)
    s["dims"] = harness.dims_of(s["wl"])
    s["dw"] = harness.dense_weights(s["w"])
    s["kv"] = harness.host_kv(s["k"], s["v"])
    return s


@pytest.fixture(scope="module")
def tiny_u():
    """The small model with norm gains drawn U(0.5, 1.5), so that a skipped gain shows."""
    return _setup("uniform")


def _run(s, dw=None, dims=None, forced=None, tokens=None, dtype=np.float32, step=None):
    ctx = s["ctx"]
    step = step or oracle.decode_step
    return step(dims or s["dims"], dw or s["dw"], copy.deepcopy(s["kv"]),
                s["tokens"] if tokens is None else tokens, ctx.copy(), s["block_tables"],
                ctx + 1, dtype, forced_topk=forced)


def _no_attention(dw):
    dw = copy.deepcopy(dw)
    for lw in dw.layers:
        lw.w_o[:] = 0
    return dw


def _f(u16):
    return bf16_to_f32(u16).astype(np.float64)


# ------------------------------------------------------------------------------ MoE branch

def check_moe_term_is_the_weighted_sum_of_experts_on_the_normed_input(s, step=None):
    """With W_o = 0 the layer adds exactly the MoE term: x1 - x0 equals the sum over route(r) of
    w_e * expert_ffn(n) with n = rmsnorm(x0) * g (composed from the pinned pieces, in fp64)."""
    d = s["dims"]
    dw = _no_attention(s["dw"])
    r = _run(s, step=step, dw=dw)
    lw = dw.layers[0]
    x0 = _f(dw.embed[s["tokens"][0]])
    n = oracle.rmsnorm(x0, _f(lw.attn_norm), d.rms_eps, np.float64)
    logits = _f(lw.w_router) @ n
    sel, w, _ = oracle.route(logits, d.top_k)
    moe = sum(w[i] * oracle.expert_ffn(n, lw.w_gate[e], lw.w_up[e], lw.w_down[e], np.float64) for i, e in enumerate(sel))
    got = r.x_layers[1][0].astype(np.float64) - x0
    tol = 1e-5 * np.abs(moe).max()
    assert np.array_equal(r.topk[0, 0], sel)
    assert np.abs(got - moe).max() <= tol
    # the plausible miswirings are far outside that tolerance
    wrong_input = sum(w[i] * oracle.expert_ffn(x0, lw.w_gate[e], lw.w_up[e], lw.w_down[e], np.float64)
                      for i, e in enumerate(sel))
    p_all = np.exp(logits - logits.max()) / np.sum(np.exp(logits - logits.max()))
    unrenormalised = sum(p_all[e] * oracle.expert_ffn(n, lw.w_gate[e], lw.w_up[e], lw.w_down[e], np.float64) for e in sel)
    unweighted = sum(oracle.expert_ffn(n, lw.w_gate[e], lw.w_up[e], lw.w_down[e], np.float64) for e in sel)
    for alt in (wrong_input, unrenormalised, unweighted):
        assert np.abs(alt - moe).max() > 100 * tol


def check_identical_experts_give_one_expert_output(s, step=None):
    """Every expert the same: whatever the routing, the renormalised weights sum to 1, so the MoE
    term is one expert's output on the normed input. A dropped, unrenormalised or doubled weight
    changes its scale; experts fed x (RMS 0.02 here) instead of n (RMS ~1) change it by orders."""
    d = s["dims"]
    dw = _no_attention(s["dw"])
    for lw in dw.layers:
        lw.w_gate[:] = lw.w_gate[3]
        lw.w_up[:] = lw.w_up[3]
        lw.w_down[:] = lw.w_down[3]
    r = _run(s, step=step, dw=dw)
    lw = dw.layers[0]
    x0 = _f(dw.embed[s["tokens"][0]])
    n = x0 / np.sqrt(np.mean(x0 * x0) + d.rms_eps) * _f(lw.attn_norm)
    # SwiGLU written out directly: W_down (SiLU(W_gate n) * (W_up n))
    g, u = _f(lw.w_gate[0]) @ n, _f(lw.w_up[0]) @ n
    one = _f(lw.w_down[0]) @ (g / (1 + np.exp(-g)) * u)
    got = r.x_layers[1][0].astype(np.float64) - x0
    assert np.abs(got - one).max() <= 1e-5 * np.abs(one).max()


def check_moe_term_is_invariant_to_scaling_the_layer_input(s, step=None):
    """RMSNorm with eps = 0 is exactly invariant to scaling its input by a power of two, so with
    W_o = 0 the MoE term of layer 0 is bitwise unchanged when the embedding row is scaled by 4;
    experts reading x instead of n would see a 4x larger input (a 16x larger SwiGLU output)."""
    dims = dataclasses.replace(s["dims"], rms_eps=0.0)
    dw = _no_attention(s["dw"])
    tok = int(s["tokens"][0])
    r1 = _run(s, step=step, dw=dw, dims=dims)
    dw4 = copy.deepcopy(dw)
    dw4.embed[tok] = f32_to_bf16(bf16_to_f32(dw.embed[tok]) * np.float32(4))
    r4 = _run(s, step=step, dw=dw4, dims=dims)
    x0 = bf16_to_f32(dw.embed[tok])
    m1 = r1.x_layers[1][0] - x0
    m4 = r4.x_layers[1][0] - np.float32(4) * x0
    assert np.array_equal(r1.topk[0], r4.topk[0])
    # x0 + moe is rounded at different magnitudes, so compare the recovered terms to fp32 rounding
    assert np.abs(m1 - m4).max() <= 4 * np.finfo(np.float32).eps * np.abs(4 * x0).max()
    assert np.abs(m1).max() > 1e3 * np.finfo(np.float32).eps * np.abs(4 * x0).max()


# ------------------------------------------------------------------------------ final norm -> lm_head

def check_logits_are_lm_head_times_final_norm(s, step=None):
    """logits = W_lm . (x_L / sqrt(mean(x_L^2) + eps) * g_f), composed from the pinned RMSNorm and
    a float64 matrix product, with the final gain drawn U(0.5, 1.5)."""
    d = s["dims"]
    r = _run(s, step=step)
    xL = r.x_final[0].astype(np.float64)
    gf = _f(s["dw"].final_norm)
    assert np.abs(gf - 1).max() > 0.1                                  # the gains really vary
    ref = _f(s["dw"].lm_head) @ oracle.rmsnorm(xL, gf, d.rms_eps, np.float64)
    tol = 1e-5 * np.abs(ref).max()
    assert np.abs(r.logits[0] - ref).max() <= tol
    no_gain = _f(s["dw"].lm_head) @ oracle.rmsnorm(xL, np.ones_like(gf), d.rms_eps, np.float64)
    no_norm = _f(s["dw"].lm_head) @ xL
    for alt in (no_gain, no_norm):
        assert np.abs(alt - ref).max() > 100 * tol


def check_one_hot_lm_head_reads_the_normed_hidden_state(s, step=None):
    """lm_head row i = the unit vector at coordinate j(i): logit i is then exactly coordinate j(i)
    of the final-normed hidden state, x_L[j] / rms(x_L) * g_f[j] (closed form, no product)."""
    d = s["dims"]
    dw = copy.deepcopy(s["dw"])
    V, H = dw.lm_head.shape
    j = np.arange(V) % H
    one = f32_to_bf16(np.float32(1.0))
    dw.lm_head[:] = 0
    dw.lm_head[np.arange(V), j] = one
    r = _run(s, step=step, dw=dw)
    xL = r.x_final[0].astype(np.float64)
    normed = xL / np.sqrt(np.mean(xL * xL) + d.rms_eps) * _f(dw.final_norm)
    assert np.abs(r.logits[0] - normed[j]).max() <= 1e-6 * np.abs(normed).max()


# ------------------------------------------------------------------------------ forced routing

def check_forced_routing_weights_are_softmax_over_the_forced_set(s, step=None):
    """A forced expert set (the near-tie replay) takes weights = the full softmax of the router
    logits renormalised over the forced set, and the MoE term uses exactly those experts and
    weights (W_o = 0, so x1 - x0 is the MoE term)."""
    d = s["dims"]
    dw = _no_attention(s["dw"])
    r0 = _run(s, step=step, dw=dw)
    order = np.argsort(-r0.router_logits[0, 0], kind="stable")
    forced_set = sorted([int(order[0]), int(order[-1])])       # the top expert and the bottom one
    assert forced_set != sorted(r0.topk[0, 0].tolist())
    r = _run(s, step=step, dw=dw, forced={(0, 0): forced_set})
    logits = r.router_logits[0, 0].astype(np.float64)
    p = np.exp(logits - logits.max())
    p /= p.sum()
    w_ref = p[forced_set] / p[forced_set].sum()
    assert np.array_equal(r.topk[0, 0], forced_set)
    assert np.abs(r.topk_weight[0, 0] - w_ref).max() <= 1e-6
    lw = dw.layers[0]
    x0 = _f(dw.embed[s["tokens"][0]])
    n = oracle.rmsnorm(x0, _f(lw.attn_norm), d.rms_eps, np.float64)
    moe = sum(w_ref[i] * oracle.expert_ffn(n, lw.w_gate[e], lw.w_up[e], lw.w_down[e], np.float64)
              for i, e in enumerate(forced_set))
    got = r.x_layers[1][0].astype(np.float64) - x0
    assert np.abs(got - moe).max() <= 1e-5 * np.abs(moe).max()
    # the unrenormalised full-softmax weights are far off
    assert np.abs(p[forced_set] - w_ref).max() > 0.1


# ------------------------------------------------------------------------------ the tests

CHECKS = [check_moe_term_is_the_weighted_sum_of_experts_on_the_normed_input, check_identical_experts_give_one_expert_output, check_moe_term_is_invariant_to_scaling_the_layer_input, check_logits_are_lm_head_times_final_norm, check_one_hot_lm_head_reads_the_normed_hidden_state, check_forced_routing_weights_are_softmax_over_the_forced_set]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__[6:])
def test_composition(tiny_u, check):
    check(tiny_u)
