"""The no-alloc decode entry point (mla_decode_paged_noalloc): the same
results as mla_decode_paged, bitwise (the same kernels and metadata), with
the split partials in the library's static device scratch.  Two calls in a
row, the second on a smaller input, check that nothing of the first call's
scratch contents leaks into the second; a call whose partials exceed the
scratch is refused before anything is launched."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, to_dev
from paged_mla_decode_03_amd import DecodeBuffers, MlaError, get_mla_metadata, mla_decode_paged, workspace_bytes
from paged_mla_decode_03_amd.binding import NOALLOC_SCRATCH_BYTES, mla_decode_paged_noalloc
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _inputs(s_q, h_q, causal, seqlens, seed):
    w = Workload("custom", batch=len(seqlens), s_q=s_q, h_q=h_q, h_kv=1, causal=causal,
                 seqlens=tuple(seqlens), num_pages=None)
    return make_inputs(w, seed, seqlens=seqlens)


def _both(inp, causal, W=None):
    w = inp.workload
    q, kv, bt, L = to_dev(inp)
    meta, ns = get_mla_metadata(L, w.s_q * w.h_q, 1, W)
    ref = DecodeBuffers(q, kv, 512, meta.shape[0])
    mla_decode_paged(q, kv, bt, L, 512, meta, ns, causal=causal, buffers=ref)
    o = torch.full_like(ref.o, 5.0)
    lse = torch.full_like(ref.lse, 5.0)
    mla_decode_paged_noalloc(q, kv, bt, L, 512, meta, ns, o, lse, causal=causal)
    torch.cuda.synchronize()
    return ref, o, lse, ns


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    # First call: 5 sequences, splits of every kind (long ones over many workers).
    big = _inputs(1, 128, False, [4000, 70, 1, 2500, 640], 11)
    ref, o, lse, ns = _both(big, False)
    assert np.diff(ns.cpu().numpy()).max() > 1
    assert torch.equal(o, ref.o) and torch.equal(lse, ref.lse)
    # Second call, smaller (fewer sequences, shorter, causal with 2 query
    # tokens -> the 128-row kernel): the scratch still holds the first call's
    # partials, which must not reach it.
    small = _inputs(2, 64, True, [300, 9], 12)
    ref2, o2, lse2, ns2 = _both(small, True, W=7)
    assert np.diff(ns2.cpu().numpy()).max() > 1
    assert torch.equal(o2, ref2.o) and torch.equal(lse2, ref2.lse)


def test_noalloc_refuses_a_call_beyond_the_scratch():
    # 256 query rows per head over many workers and sequences: more than 64 MiB of partials.
    B, W = 300, 256
    assert workspace_bytes(B, 2, 128, 1, 512, W) > NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 2, 128, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 64, 1, 576), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    L = torch.full((B,), 5, dtype=torch.int32, device=DEV)
    meta = torch.zeros((W, 8), dtype=torch.int32, device=DEV)
    ns = torch.zeros((B + 1,), dtype=torch.int32, device=DEV)
    o = torch.full((B, 2, 128, 512), 5.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, 128, 2), 5.0, dtype=torch.float32, device=DEV)
    with pytest.raises(MlaError) as err:
        mla_decode_paged_noalloc(q, kv, bt, L, 512, meta, ns, o, lse, causal=True)
    assert err.value.status == -3
    torch.cuda.synchronize()
    assert (o.float() == 5.0).all() and (lse == 5.0).all()
