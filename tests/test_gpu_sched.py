"""The device scheduler against the CPU reference of the same split rule:
both outputs must be equal bit for bit."""
import numpy as np
import pytest
import torch

from oracle.sched_ref import split_rule
from paged_mla_decode_03_amd import fixed_overhead_pages, get_mla_metadata, num_workers
from workloads import WORKLOADS, draw_seqlens

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _check(seqlens, rows, h_kv, W=None):
    L = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    W = W or num_workers(rows, h_kv)
    meta, ns = get_mla_metadata(L, rows, h_kv, W)
    torch.cuda.synchronize()
    ref_meta, ref_ns = split_rule(seqlens, W, fixed_overhead_pages())
    np.testing.assert_array_equal(meta.cpu().numpy(), ref_meta)
    np.testing.assert_array_equal(ns.cpu().numpy(), ref_ns)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_metadata_bit_exact(name):
    w = WORKLOADS[name]
    for seed in (0, 1, 2):
        L = draw_seqlens(w, np.random.Generator(np.random.PCG64(seed)))
        _check([int(x) for x in L], w.rows_per_kv, w.h_kv)


@pytest.mark.parametrize("seqlens,W", [
    ([0, 1, 63, 64, 65, 131072], None),
    ([0, 0, 0], 7),
    ([5] * 3000, None),              # batch larger than the scheduler's workgroup
    ([1], 1),
    ([100000, 3, 0, 5000], 4096),
    ([64 * (i % 37) + i % 5 for i in range(256)], None),    # exactly one workgroup of sequences
    ([64 * (i % 41) + i % 7 for i in range(257)], 300),     # one past it
    ([(i * 7919) % 20000 for i in range(1000)], 333),       # four chunks, ragged lengths and zeros
])
def test_edge_metadata_bit_exact(seqlens, W):
    _check(seqlens, 128, 1, W)


def test_num_workers_uses_all_cus():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert num_workers(64, 1) == cus
    assert num_workers(128, 1) == cus // 2      # two 64-row blocks
    assert num_workers(256, 1) == cus // 2      # two 128-row blocks
    assert num_workers(320, 1) == cus // 3
