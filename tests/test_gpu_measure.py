"""The measurement helpers run through the C ABI and return sane figures
(they time hardware rates; no oracle applies)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("waves", [4, 8])
def test_lds_read_rate_runs(waves):
    from paged_mla_decode_03_amd.binding import LDS_READ_KINDS, lds_read_rate
    dev = torch.device("cuda", 0)
    for kind in LDS_READ_KINDS:
        cyc = lds_read_rate(kind, waves, 16, 8, dev)
        torch.cuda.synchronize()
        c = cyc.cpu()
        assert bool((c > 0).all()), (kind, c)
        per_read = float(c.double().median()) / (64 * 16)
        # A read of a wave takes at least a few cycles and far less than a microsecond.
        assert 1.0 < per_read < 2000.0, (kind, per_read)


def test_stream_read_runs():
    from paged_mla_decode_03_amd.binding import stream_read
    src = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    stream_read(src)
    torch.cuda.synchronize()
