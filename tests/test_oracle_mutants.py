"""The composition pins must catch plausible wiring mistakes in the oracle's decode step.

Each case plants one mistake into a copy of the oracle's decode-step source (on the CPU, in
memory; the oracle on disk is untouched), runs every composition check of
test_oracle_composition.py against the mutated step, and requires at least one check to fail.
"""

import inspect
import types

import pytest

import oracle.decode
from tests import test_oracle_composition as comp

MUTANTS = {
    "experts fed x instead of the normed input":
        ("moe += we * expert_ffn(n, g_, u_, d_, dtype)", "moe += we * expert_ffn(x[b], g_, u_, d_, dtype)"),
    "expert weight dropped":
        ("moe += we * expert_ffn(n,", "moe += expert_ffn(n,"),
    "forced-set weights not renormalised":
        ("                wsel = e / np.sum(e, dtype=dtype)", "                wsel = e"),
    "final gain skipped":
        ("rmsnorm(x[b], gf, dims.rms_eps, dtype)", "rmsnorm(x[b], np.ones_like(gf), dims.rms_eps, dtype)"),
    "final norm skipped":
        ("logits[b, s:e] = (wl @ n_final[b])", "logits[b, s:e] = (wl @ x[b])"),
    "layer gain skipped":
        ("n = rmsnorm(x[b], _dec(lw.attn_norm, dtype), dims.rms_eps, dtype)",
         "n = rmsnorm(x[b], np.ones(H, dtype), dims.rms_eps, dtype)"),
}


def _mutant_step(old, new):
    src = inspect.getsource(oracle.decode)
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle._decode_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<oracle.decode mutant>", "exec"), mod.__dict__)
    return mod.decode_step


@pytest.fixture(scope="module")
def tiny_u():
    return comp._setup("uniform")


def test_unmutated_step_passes_every_check(tiny_u):
    step = _mutant_step("def decode_step(", "def decode_step(")
    for check in comp.CHECKS:
        check(tiny_u, step)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tiny_u, name):
    step = _mutant_step(*MUTANTS[name])
    failed = []
    for check in comp.CHECKS:
        try:
            check(tiny_u, step)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no composition check caught: {name}"
