"""Host-side checks of the seeded input generators (no method arithmetic in them)."""


def test_refill_sequence_reshuffles_the_slots_own_pages():
    """Slot refill (continuous batching): the slot keeps exactly its own pages in a new seeded
    order, only the pages covering the new prompt get fresh K/V (other slots' pages untouched), and
    a slot too small for the new sequence is refused."""
    import numpy as np
    import pytest
    import torch
    from decode_megakernel_03_amd import synth
    wl = synth.workload("tiny", batch=3, ragged=(17, 200))
    ctx = synth.context_lengths(wl)
    bt, num_pages = synth.make_block_tables(ctx, 16, wl.page_size)
    k, v = synth.make_kv(wl, num_pages)
    k0 = [t.clone() for t in k]
    row, tok = synth.refill_sequence(wl, k, v, bt, 1, 30, 8, seed=9)
    own = bt[1][bt[1] >= 0]
    assert sorted(row[row >= 0].tolist()) == sorted(own.tolist()) and (row[len(own):] == -1).all()
    row2, tok2 = synth.refill_sequence(wl, [t.clone() for t in k], [t.clone() for t in v], bt, 1, 30, 8, seed=9)
    assert np.array_equal(row, row2) and tok == tok2 and 0 <= tok < wl.vocab          # seeded
    need = -(-(30 + 8) // wl.page_size)
    changed = {int(p) for p in range(num_pages) if not torch.equal(k[0][p], k0[0][p])}
    assert changed == set(row[:need].tolist())
    with pytest.raises(ValueError):
        synth.refill_sequence(wl, k, v, bt, 1, 200, 8, seed=9)
