"""Pins of the oracle's prefill (``oracle.prefill``): a whole prompt in one causal forward pass.

The decode step is pinned piece by piece and as a composition elsewhere. The prefill is a second
formulation of the same definition (every projection over all positions at once, a masked score
matrix, each expert over the block of positions routed to it), pinned here against:

* the decode step run one position at a time (what a prefill must equal, position by position:
  the pages' engine decodes every generated token with the same layers it prefills with);
* itself on the prompt split in two (the second part continuing from the cache the first wrote);
* causality: changing one prompt token changes nothing at earlier positions and does change its
  own position;
* a one-position prefill, which is a decode step at that position.

Planted mistakes (mask off by one, RoPE at the wrong positions, K/V written after attending, the
causal mask dropped, experts weighted without their router weight) must each fail a pin.
"""

import copy
import inspect
import types

import numpy as np
import pytest

import oracle
import oracle.prefill
from decode_megakernel_03_amd import synth
from tests import harness

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

N = 19          # prompt positions: several 8-row chunks and a ragged tail when run on the GPU


def _setup(start, n=N, seed=3):
    wl = synth.workload("tiny", steps=n + 8)
    s = harness.tiny_setup(wl, ctx=[start], gains="uniform")
    s["dims"] = harness.dims_of(wl)
    s["dw"] = harness.dense_weights(s["w"])
    s["kv"] = harness.host_kv(s["k"], s["v"])
    s["prompt"] = np.random.default_rng(seed).integers(0, wl.vocab, n).astype(np.int64)
    s["start"] = start
    return s


@pytest.fixture(scope="module", params=[0, 21], ids=["from-position-0", "after-21-cached"])
def tiny(request):
    return _setup(request.param)


def _sequential(s, tokens, start):
    """The decode step, one position at a time, on a copy of the cache."""
    kv = copy.deepcopy(s["kv"])
    bt = s["block_tables"]
    out = []
    for i, t in enumerate(tokens):
        p = start + i
        out.append(oracle.decode_step(s["dims"], s["dw"], kv, [int(t)], np.array([p]), bt, np.array([p + 1])))
    return kv, out


def _prefill(s, tokens, start, fn=None, kv=None, **kw):
    kv = copy.deepcopy(s["kv"]) if kv is None else kv
    res = (fn or oracle.prefill.prefill)(s["dims"], s["dw"], kv, tokens, s["block_tables"][0], start, **kw)
    return kv, res


def _kv_rows(s, kv, positions):
    """K and V of every layer at the given positions: [L, 2, len(positions), Hkv, D] bf16 codes."""
    bt = s["block_tables"][0]
    ps = s["dims"].page_size
    rows = []
    for l in range(s["dims"].n_layers):
        rows.append([np.stack([c[l][bt[p // ps], :, p % ps, :] for p in positions]) for c in (kv.k, kv.v)])
    return np.asarray(rows)


def check_equals_sequential(s, fn=None):
    start, tokens = s["start"], s["prompt"]
    kv_a, res = _prefill(s, tokens, start, fn, all_logits=True)
    kv_b, seq = _sequential(s, tokens, start)
    pos = list(range(start, start + len(tokens)))
    # routing: the same experts at every layer and position (no near tie in these inputs)
    for i, r in enumerate(seq):
        assert np.array_equal(res.topk[:, i, :], r.topk[:, 0, :]), f"routing differs at position {start + i}"
    assert res.margin.min() > 1e-3
    # K/V written: at most one bf16 step apart (fp32 sums in another order)
    bad = harness.bf16_step_mismatch(_kv_rows(s, kv_a, pos), _kv_rows(s, kv_b, pos))
    assert not bad.any(), f"{bad.sum()} K/V entries differ by more than one bf16 step"
    # logits of every position and the final residual stream
    ref = np.stack([r.logits[0] for r in seq])
    assert np.max(np.abs(res.logits - ref)) <= 1e-4 * max(1.0, np.max(np.abs(ref)))
    xs = np.stack([r.x_final[0] for r in seq])
    assert np.allclose(res.x_final, xs, rtol=1e-4, atol=1e-5)


def check_split_prompt(s, fn=None):
    start, tokens = s["start"], s["prompt"]
    a = 7
    kv_w, whole = _prefill(s, tokens, start, fn)
    kv_s, _ = _prefill(s, tokens[:a], start, fn)
    kv_s, tail = _prefill(s, tokens[a:], start + a, fn, kv=kv_s)
    pos = list(range(start, start + len(tokens)))
    assert not harness.bf16_step_mismatch(_kv_rows(s, kv_w, pos), _kv_rows(s, kv_s, pos)).any()
    assert np.max(np.abs(whole.logits - tail.logits)) <= 1e-4 * max(1.0, np.max(np.abs(whole.logits)))


def check_causal(s, fn=None):
    start, tokens = s["start"], s["prompt"]
    j = 11
    other = tokens.copy()
    other[j] = (other[j] + 517) % s["dims"].vocab
    kv_a, ra = _prefill(s, tokens, start, fn, all_logits=True)
    kv_b, rb = _prefill(s, other, start, fn, all_logits=True)
    before = list(range(start, start + j))
    assert np.array_equal(_kv_rows(s, kv_a, before), _kv_rows(s, kv_b, before))
    assert np.allclose(ra.logits[:j], rb.logits[:j], rtol=0, atol=1e-6)
    # and the changed position itself moves (its embedding differs)
    assert not np.array_equal(_kv_rows(s, kv_a, [start + j]), _kv_rows(s, kv_b, [start + j]))
    assert np.max(np.abs(ra.logits[j] - rb.logits[j])) > 1e-3


def check_one_position(s, fn=None):
    start, tokens = s["start"], s["prompt"][:1]
    kv_a, res = _prefill(s, tokens, start, fn)
    kv_b, seq = _sequential(s, tokens, start)
    assert np.array_equal(res.topk[:, 0, :], seq[0].topk[:, 0, :])
    assert np.max(np.abs(res.logits - seq[0].logits[0])) <= 1e-4 * max(1.0, np.max(np.abs(seq[0].logits)))
    assert not harness.bf16_step_mismatch(_kv_rows(s, kv_a, [start]), _kv_rows(s, kv_b, [start])).any()


CHECKS = [check_equals_sequential, check_split_prompt, check_causal, check_one_position]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_prefill_pins(tiny, check):
    check(tiny)


MUTANTS = {
    "mask off by one (a position does not see its own key)":
        ("visible = np.arange(T)[None, :] <= pos[:, None]", "visible = np.arange(T)[None, :] < pos[:, None] + (pos[:, None] == 0)"),
    "no causal mask":
        ("s = np.where(visible, s, dtype(-np.inf))", "s = s"),
    "RoPE at positions counted from the prompt start":
        ("k_new = _rope_rows(qkv[:, hq * D: (hq + hkv) * D].reshape(n, hkv, D), pos,",
         "k_new = _rope_rows(qkv[:, hq * D: (hq + hkv) * D].reshape(n, hkv, D), pos - start,"),
    "K/V gathered before the prompt's rows are written":
        ("        kk = _dec(gather_paged(kv.k[l], block_table, T, dims.page_size), dtype)   # [T, Hkv, D]",
         "        kk = _dec(gather_paged(kv.k[l], block_table, T, dims.page_size), dtype) * 0 + _stale_k(kv, l, block_table, T, dims, dtype, pos)"),
    "expert output without its router weight":
        ("moe[rows] += wsel[rows, e_id][:, None] * (hmid @ _dec(d_, dtype).T)", "moe[rows] += (hmid @ _dec(d_, dtype).T)"),
}

_STALE = '''
def _stale_k(kv, l, block_table, T, dims, dtype, pos):
    k = _dec(gather_paged(kv.k[l], block_table, T, dims.page_size), dtype).copy()
    k[pos] = 0.0                       # the prompt's own keys as they were before this call
    return k
'''


def _mutant(old, new):
    src = inspect.getsource(oracle.prefill)
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle._prefill_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new) + _STALE, "<oracle.prefill mutant>", "exec"), mod.__dict__)
    return mod.prefill


@pytest.fixture(scope="module")
def tiny_cached():
    return _setup(21)


def test_unmutated_prefill_passes_every_pin(tiny_cached):
    fn = _mutant("def prefill(", "def prefill(")
    for check in CHECKS:
        check(tiny_cached, fn)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(tiny_cached, name):
    fn = _mutant(*MUTANTS[name])
    failed = []
    for check in CHECKS:
        try:
            check(tiny_cached, fn)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no pin caught: {name}"
