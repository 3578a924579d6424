"""Host logic of the parity harness: layer-ordered near-tie replay (no GPU)."""

import numpy as np
import pytest

from tests import harness


class _Res:
    def __init__(self, topk, margin, router_logits):
        self.topk, self.margin, self.router_logits = topk, margin, router_logits


E = 12


def _logits(L, B, flip_layer, flip_margin):
    """Router logits whose top-4 is experts 0..3 (ranks 1..4 in that order), expert 4 ranked 5th
    (margin r_(4) - r_(5) = 0.5, or flip_margin at (flip_layer, token 0)), the rest far below."""
    r = np.full((L, B, E), -10.0) - np.arange(E) * 0.01
    r[:, :, :4] = [4.0, 3.0, 2.0, 1.0]
    r[:, :, 4] = 0.5
    r[flip_layer, 0, 4] = 1.0 - flip_margin
    return r


def _fake_oracle(L, B, flip_layer, flip_margin, gpu_set=(0, 1, 2, 4)):
    """An 'oracle' whose sets after a forced flip at flip_layer follow the GPU's trajectory, and
    differ from it (by several experts) otherwise, like a residual stream that diverged."""
    gpu = np.tile(np.arange(4, dtype=np.int32), (L, B, 1))
    gpu[flip_layer, 0] = list(gpu_set)                    # the GPU's side of the near-tie
    for l in range(flip_layer + 1, L):
        gpu[l, 0] = [8, 9, 10, 11]

    def run(forced):
        topk = np.tile(np.arange(4, dtype=np.int32), (L, B, 1))
        margin = np.full((L, B), 0.5)
        margin[flip_layer, 0] = flip_margin
        if forced and (flip_layer, 0) in forced:
            topk[flip_layer, 0] = forced[(flip_layer, 0)]
            for l in range(flip_layer + 1, L):
                topk[l, 0] = [8, 9, 10, 11]
        return _Res(topk, margin, _logits(L, B, flip_layer, flip_margin))
    return run, gpu


def test_near_tie_then_divergence_is_accepted():
    run, gpu = _fake_oracle(L=6, B=2, flip_layer=2, flip_margin=5e-5)
    ref, forced = harness.replay_near_ties(run, gpu, 1e-4)
    assert forced == {(2, 0): [0, 1, 2, 4]}
    assert np.array_equal(ref.topk, gpu)


def test_real_mismatch_raises():
    run, gpu = _fake_oracle(L=6, B=2, flip_layer=2, flip_margin=0.05)
    with pytest.raises(harness.RoutingMismatch, match="layer 2 token 0"):
        harness.replay_near_ties(run, gpu, 1e-4)


def test_two_swaps_is_not_a_near_tie():
    run, gpu = _fake_oracle(L=4, B=1, flip_layer=1, flip_margin=1e-6)
    gpu[1, 0] = [0, 1, 6, 7]
    with pytest.raises(harness.RoutingMismatch):
        harness.replay_near_ties(run, gpu, 1e-4)


def test_swap_with_a_far_rank_is_not_a_near_tie():
    """The k/k+1 margin is tiny, but the GPU dropped rank 4 for the rank-9 expert (not rank 5)."""
    run, gpu = _fake_oracle(L=4, B=1, flip_layer=1, flip_margin=1e-6, gpu_set=(0, 1, 2, 8))
    with pytest.raises(harness.RoutingMismatch, match="ranks k, k\\+1 = 3, 4"):
        harness.replay_near_ties(run, gpu, 1e-4)


def test_dropping_a_top_rank_is_not_a_near_tie():
    """The GPU kept ranks 4 and 5 but dropped rank 1: one expert swapped, small margin, still wrong."""
    run, gpu = _fake_oracle(L=4, B=1, flip_layer=1, flip_margin=1e-6, gpu_set=(1, 2, 3, 4))
    with pytest.raises(harness.RoutingMismatch):
        harness.replay_near_ties(run, gpu, 1e-4)


def test_agreement_needs_one_oracle_run():
    calls = []

    def run(forced):
        calls.append(forced)
        return _Res(np.zeros((3, 1, 2), np.int32) + [0, 1], np.ones((3, 1)), np.zeros((3, 1, 4)))
    ref, forced = harness.replay_near_ties(run, np.zeros((3, 1, 2), np.int32) + [0, 1], 1e-4)
    assert forced == {} and calls == [None]


def test_bf16_step_mismatch_accepts_exactly_one_step():
    """Neighbouring bf16 patterns pass (also across a binade boundary); two steps, a sign flip of
    a sizeable value, or a change beyond the noise floor near zero fail."""
    import oracle
    base = oracle.f32_to_bf16(np.array([1.0, 1.0, 2.0, -3.0, 1e-7, 0.5, 1e-7], np.float32))
    other = base.copy()
    other[0] += 1                                        # one step up
    other[1] += 2                                        # two steps up
    other[2] -= 1                                        # 2.0 -> 1.9921875: one step across the binade
    other[3] = oracle.f32_to_bf16(np.float32(3.0))       # sign flip of a sizeable value
    other[4] = oracle.f32_to_bf16(np.float32(-5e-6))     # near zero, within the 1e-5 floor
    other[5] = base[5] + 1                               # one step
    other[6] = oracle.f32_to_bf16(np.float32(3e-5))      # near zero but beyond the floor
    bad = harness.bf16_step_mismatch(other, base)
    assert bad.tolist() == [False, True, False, True, False, False, True]
