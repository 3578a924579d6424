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
