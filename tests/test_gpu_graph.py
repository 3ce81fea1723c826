"""The decode under HIP graph capture, as a serving loop replays it: the
decode and combine launches of mla_decode_paged (and of the no-alloc entry,
whose callers include code under capture) captured into a graph and replayed
several times, with the program's own eager work and synchronisations
between the replays.  Every replay must equal the eager result bit for bit
(the same kernels on the same inputs, a fixed order of every sum), and the
eager result the oracle."""
import pytest
import torch

from gpu_helpers import DEV, compare, oracle
from paged_mla_decode_03_amd import DecodeBuffers, get_mla_metadata, mla_decode_paged
from paged_mla_decode_03_amd import workspace_bytes
from paged_mla_decode_03_amd.binding import NOALLOC_SCRATCH_BYTES, mla_decode_paged_noalloc
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [(1, 128, False, [100, 5000, 7, 640]),    # 64-row kernel, split and whole sequences
         (2, 128, True, [300, 70, 9])]             # 128-row kernel, causal


def _inputs(s_q, h_q, causal, seqlens, num_workers=None):
    w = Workload("custom", batch=len(seqlens), s_q=s_q, h_q=h_q, h_kv=1, causal=causal, seqlens=tuple(seqlens),
                 num_pages=None)
    inp = make_inputs(w, 11, seqlens=seqlens)
    q, kv, bt, L = (t.to(DEV) for t in (inp.q, inp.kvcache, inp.block_table, inp.cache_seqlens))
    meta, ns = get_mla_metadata(L, s_q * h_q, 1, num_workers)
    return inp, q, kv, bt, L, meta, ns


def _replays_equal(launch, outs, eager):
    """Capture launch() (after one warm call on a side stream), then replay
    four times, clearing the outputs eagerly before each replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for i in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("s_q,h_q,causal,seqlens", CASES)
def test_decode_graph_replays_equal_eager(s_q, h_q, causal, seqlens):
    inp, q, kv, bt, L, meta, ns = _inputs(s_q, h_q, causal, seqlens)
    buf = DecodeBuffers(q, kv, 512, meta.shape[0])
    mla_decode_paged(q, kv, bt, L, 512, meta, ns, causal=causal, buffers=buf)
    torch.cuda.synchronize()
    eager = (buf.o.clone(), buf.lse.clone())
    O, LSE = oracle(inp)
    compare(eager[0].float().cpu().double().numpy(), eager[1].cpu().double().numpy(), O, LSE, label="eager")
    _replays_equal(lambda: mla_decode_paged(q, kv, bt, L, 512, meta, ns, causal=causal, buffers=buf),
                   (buf.o, buf.lse), eager)


@pytest.mark.parametrize("s_q,h_q,causal,seqlens", CASES)
def test_noalloc_graph_replays_equal_eager(s_q, h_q, causal, seqlens):
    # 64 workers keep the split partials inside the library's static scratch
    # (at 256 query rows per head the default count would not fit).
    inp, q, kv, bt, L, meta, ns = _inputs(s_q, h_q, causal, seqlens, num_workers=64)
    assert workspace_bytes(len(seqlens), s_q, h_q, 1, 512, 64) <= NOALLOC_SCRATCH_BYTES
    o = torch.empty((len(seqlens), s_q, h_q, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((len(seqlens), h_q, s_q), dtype=torch.float32, device=DEV)
    mla_decode_paged_noalloc(q, kv, bt, L, 512, meta, ns, o, lse, causal=causal)
    torch.cuda.synchronize()
    eager = (o.clone(), lse.clone())
    ref = DecodeBuffers(q, kv, 512, meta.shape[0])
    mla_decode_paged(q, kv, bt, L, 512, meta, ns, causal=causal, buffers=ref)
    torch.cuda.synchronize()
    assert torch.equal(ref.o, eager[0]) and torch.equal(ref.lse, eager[1])
    _replays_equal(lambda: mla_decode_paged_noalloc(q, kv, bt, L, 512, meta, ns, o, lse, causal=causal),
                   (o, lse), eager)
