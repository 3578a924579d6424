"""Host logic of the parity harness: layer-ordered near-tie replay (no GPU)."""

import numpy as np
import pytest

from tests import harness


class _Res:
    def __init__(self, topk, margin):
        self.topk, self.margin = topk, margin


def _fake_oracle(L, B, flip_layer, flip_margin):
    """An 'oracle' whose sets after a forced flip at flip_layer follow the GPU's trajectory, and
    differ from it (by several experts) otherwise, like a residual stream that diverged."""
    gpu = np.tile(np.arange(4, dtype=np.int32), (L, B, 1))
    gpu[flip_layer, 0] = [0, 1, 2, 5]                     # the GPU's side of the near-tie
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
        return _Res(topk, margin)
    return run, gpu


def test_near_tie_then_divergence_is_accepted():
    run, gpu = _fake_oracle(L=6, B=2, flip_layer=2, flip_margin=5e-5)
    ref, forced = harness.replay_near_ties(run, gpu, 1e-4)
    assert forced == {(2, 0): [0, 1, 2, 5]}
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


def test_agreement_needs_one_oracle_run():
    calls = []

    def run(forced):
        calls.append(forced)
        return _Res(np.zeros((3, 1, 2), np.int32) + [0, 1], np.ones((3, 1)))
    ref, forced = harness.replay_near_ties(run, np.zeros((3, 1, 2), np.int32) + [0, 1], 1e-4)
    assert forced == {} and calls == [None]
