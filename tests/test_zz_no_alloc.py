"""The allocation-free entry point mk_handoff_litmus_noalloc against mk_handoff_litmus, through the
C ABI: the same results (bit-exact integers) on two calls in a row, the second with a smaller input
(fewer rounds, fewer words, fewer workgroups), so that stale contents of the shared scratch array
from the first call would show; and sizes beyond the array are refused."""

import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def test_noalloc_matches_the_allocating_entry_point():
    from decode_megakernel_03_amd import mk
    torch.zeros(1, device="cuda")              # the GPU is initialised as in the other tests
    for rounds, words, wgs in ((800, mk.MK_LITMUS_NOALLOC_MAX_WORDS, 512), (300, 1000, 128)):
        print(f"litmus rounds {rounds} words {words} workgroups {wgs}", flush=True)
        ref = mk.mk_handoff_litmus(rounds, words, wgs)
        got = mk.mk_handoff_litmus_noalloc(rounds, words, wgs)
        print(f"  allocating {ref}, allocation-free {got}", flush=True)
        assert ref[0] == mk.MK_OK and got[0] == mk.MK_OK
        assert got == ref
        assert got[1] == 0 and got[2] == rounds * words * (wgs - 1)


def test_noalloc_refuses_sizes_beyond_the_scratch_array():
    from decode_megakernel_03_amd import mk
    st, _, _ = mk.mk_handoff_litmus_noalloc(10, mk.MK_LITMUS_NOALLOC_MAX_WORDS + 1, 64)
    assert st == mk.MK_ERR_INVALID_ARG
    assert mk.mk_handoff_litmus_noalloc(0, 16, 64)[0] == mk.MK_ERR_INVALID_ARG
    assert mk.mk_handoff_litmus_noalloc(10, 16, 1)[0] == mk.MK_ERR_INVALID_ARG
    # and the array still works afterwards
    assert mk.mk_handoff_litmus_noalloc(20, 64, 64) == (mk.MK_OK, 0, 20 * 64 * 63)
