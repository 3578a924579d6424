"""GPU checks of the library's measurement helper."""

import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def test_stream_read_bandwidth_is_plausible():
    """256 MiB streamed by the library's read kernel: a bandwidth between 0.5 and 10 TB/s (MI355X
    HBM3E peaks at 8 TB/s), and the buffer is left unchanged."""
    from decode_megakernel_03_amd import mk
    print("test_stream_read_bandwidth_is_plausible: 256 MiB, 3 passes", flush=True)
    x = torch.arange(64 << 20, dtype=torch.int32, device="cuda")
    ref = x.clone()
    bw = mk.mk_stream_read_bandwidth(x.data_ptr(), x.numel() * 4, 3)
    torch.cuda.synchronize()
    assert 0.5e12 < bw < 10e12, bw
    assert torch.equal(x, ref)


def test_handoff_litmus_across_xcds():
    """The step kernel's hand-off protocol (write-through stores, wait, barrier, relaxed counter add;
    consumers poll, barrier, read with write-through-coherent loads) on 512 co-resident workgroups
    spread over all 8 XCDs: 2000 rounds with a different producer each round, 4096 words each,
    255+ consumers per round; not one consumer may read a stale word."""
    from decode_megakernel_03_amd import mk
    print("test_handoff_litmus_across_xcds: 2000 rounds x 4096 words, 512 workgroups", flush=True)
    st, stale, checked = mk.mk_handoff_litmus(2000, 4096, 512)
    print(f"  status {st}, stale {stale} of {checked} words read", flush=True)
    assert st == mk.MK_OK
    assert checked == 2000 * 4096 * 511
    assert stale == 0


def test_handoff_litmus_rejects_bad_arguments():
    from decode_megakernel_03_amd import mk
    assert mk.mk_handoff_litmus(0, 16, 64)[0] == mk.MK_ERR_INVALID_ARG
    assert mk.mk_handoff_litmus(10, 0, 64)[0] == mk.MK_ERR_INVALID_ARG
    assert mk.mk_handoff_litmus(10, 16, 1)[0] == mk.MK_ERR_INVALID_ARG
    assert mk.mk_handoff_litmus(10, 16, 1 << 20)[0] == mk.MK_ERR_INVALID_ARG   # cannot all be resident
