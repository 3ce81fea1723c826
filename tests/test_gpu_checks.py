"""The table checker (mla_check_inputs), the opt-in debug path in front of
the decode, and the decode kernels' own guard against a bad page id: an id
outside [0, num_pages) is staged as a page of zeros, so the kernels never
form an address outside the cache, and other sequences are unaffected."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, run_gpu, to_dev
from paged_mla_decode_03_amd import (DecodeBuffers, MlaError, check_inputs, get_mla_metadata, mla_decode_paged,
                                     set_debug_checks)
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _custom(h_q, seqlens, seed, s_q=1, **kw):
    w = Workload("custom", batch=len(seqlens), s_q=s_q, h_q=h_q, h_kv=1, causal=False,
                 seqlens=tuple(seqlens), num_pages=None)
    return make_inputs(w, seed, seqlens=seqlens, **kw)


def _check(bt, L, num_pages):
    res = check_inputs(bt.to(DEV), L.to(DEV), num_pages)
    torch.cuda.synchronize()
    return res.cpu().tolist()


def test_checker_accepts_valid_tables():
    inp = _custom(16, [0, 37, 130, 64, 1], 1, extra_pages=3)
    assert _check(inp.block_table, inp.cache_seqlens, inp.kvcache.shape[0]) == [0, -1, -1, 0]


def test_checker_finds_each_kind_of_bad_entry():
    inp = _custom(16, [37, 130, 64, 200], 2)
    P = inp.kvcache.shape[0]
    mp = inp.block_table.shape[1]
    for b, j, value, first in [(1, 2, P, (1, 2)), (2, 0, -1, (2, 0)), (0, 0, 1 << 30, (0, 0)),
                               (3, 3, -7, (3, 3))]:
        bt = inp.block_table.clone()
        bt[b, j] = value
        assert _check(bt, inp.cache_seqlens, P) == [1, first[0], first[1], 0], (b, j, value)
    # lengths: negative, and more tokens than the table row maps
    for b, value in [(1, -1), (2, 64 * mp + 1)]:
        L = inp.cache_seqlens.clone()
        L[b] = value
        assert _check(inp.block_table, L, P) == [1, b, -1, 0], (b, value)
    # padding past ceil(L/64) is never read, so it is not checked
    bt = inp.block_table.clone()
    assert (bt[0, 1:] == -1).all()
    assert _check(bt, inp.cache_seqlens, P)[0] == 0
    # two bad entries: both counted, the first one named
    bt[3, 1] = P + 5
    bt[1, 0] = -3
    assert _check(bt, inp.cache_seqlens, P) == [2, 1, 0, 0]


def test_checker_on_a_large_table():
    """Many sequences and blocks: the one workgroup loops over all of them."""
    inp = make_inputs("var_len", 0)
    bt, L = inp.block_table, inp.cache_seqlens
    P = inp.kvcache.shape[0]
    assert _check(bt, L, P)[0] == 0
    b = int(np.argmax(L.numpy()))
    j = int((L[b] - 1) // 64)
    bt = bt.clone()
    bt[b, j] = P
    assert _check(bt, L, P) == [1, b, j, 0]


def test_debug_checks_refuse_a_bad_table_and_launch_nothing():
    inp = _custom(128, [300, 70, 5], 3)
    q, kv, bt, L = to_dev(inp)
    meta, ns = get_mla_metadata(L, 128, 1)
    good = DecodeBuffers(q, kv, 512, meta.shape[0])
    mla_decode_paged(q, kv, bt, L, 512, meta, ns, buffers=good)
    bad_bt = bt.clone()
    bad_bt[0, 2] = kv.shape[0]
    buf = DecodeBuffers(q, kv, 512, meta.shape[0])
    buf.o.fill_(3.0)
    set_debug_checks(True)
    try:
        with pytest.raises(MlaError) as err:
            mla_decode_paged(q, kv, bad_bt, L, 512, meta, ns, buffers=buf)
        assert err.value.status == -6
        torch.cuda.synchronize()
        assert (buf.o.float() == 3.0).all()          # nothing was launched
        # a valid table passes the checks and gives the same result
        mla_decode_paged(q, kv, bt, L, 512, meta, ns, buffers=buf)
        torch.cuda.synchronize()
        assert torch.equal(buf.o, good.o) and torch.equal(buf.lse, good.lse)
    finally:
        set_debug_checks(False)


@pytest.mark.parametrize("s_q", [1, 2])
def test_bad_page_id_reads_zeros_and_leaves_other_sequences_alone(s_q):
    """Without the checks, a page id past the cache is staged as zeros (an
    empty buffer resource): no fault, a finite result, and the sequences
    whose tables are valid come out bitwise as with a valid table.  s_q = 2
    (256 query rows) runs the 128-row kernel, s_q = 1 the 64-row one."""
    inp = _custom(128, [300, 70, 130], 4, s_q=s_q)
    ref = run_gpu(inp)
    P = inp.kvcache.shape[0]
    inp.block_table[1, 0] = P + 1000
    inp.block_table[2, 2] = -5
    got = run_gpu(inp)
    assert np.isfinite(got[0]).all()
    assert np.array_equal(got[0][0], ref[0][0]) and np.array_equal(got[1][0], ref[1][0])
