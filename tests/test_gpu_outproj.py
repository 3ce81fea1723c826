"""The output projection over all heads, u_t = W^O [o_{t,1}; ...; o_{t,n_h}],
on the GPU (mla_outproj through the C ABI) against the oracle's
out_proj_ref.  Each element within 2^-8 of its magnitude plus 10^-3 of the
output's RMS: one bf16 rounding of the fp32 sum (half an ulp is at most
2^-9 of the magnitude) plus fp32 accumulation over up to 16384 products."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV
from oracle.mla_oracle import out_proj_ref
from paged_mla_decode_03_amd import library, outproj
from workloads import bf16_normal

pytestmark = pytest.mark.gpu


def _inputs(T, h, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    o = bf16_normal(rng, (T, h, 128))
    w = (bf16_normal(rng, (n, h * 128)).float() / float(np.sqrt(h * 128))).to(torch.bfloat16)
    return o, w


def _check(u, U, label):
    u = u.float().cpu().double().numpy()
    rms = float(np.sqrt(np.mean(U ** 2)))
    d = np.abs(u - U)
    bound = 2.0 ** -8 * np.abs(U) + 1e-3 * rms
    print(f"[parity] outproj {label}: max|du| {d.max():.3e}, rms(U) {rms:.3f}", flush=True)
    assert (d <= bound).all(), f"{label}: max excess {(d - bound).max()}"


def _splits(T, h, n):
    return int(library().mla_outproj_workspace_bytes(T, h * 128, n)) // (4 * T * n)


@pytest.mark.parametrize("T,h,n", [
    (1, 1, 128),        # one token, one head
    (5, 4, 256),        # ragged token chunk
    (64, 16, 512),      # one full token chunk
    (130, 8, 384),      # three token chunks, the last ragged
    (200, 128, 256),    # many heads (K = 16384) over few output columns
])
def test_outproj_small(T, h, n):
    o, w = _inputs(T, h, n, seed=T + h + n)
    u = outproj(o.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    _check(u, out_proj_ref(o, w), f"T={T} h={h} n={n} splits={_splits(T, h, n)}")


@pytest.mark.parametrize("T", [64, 264])
def test_outproj_full_width_sampled(T):
    """128 heads into d_model = 16384 (the whole projection, 537 MB of W^O),
    the token counts of the mem_bound and causal_sq2 decode steps; the
    oracle checks 192 sampled output columns (every token), the GPU computes
    them all; both the split-K path (T = 64) and the direct one (T = 264)."""
    h, n = 128, 16384
    o, w = _inputs(T, h, n, seed=T)
    u = outproj(o.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(T).choice(n, size=192, replace=False))
    U = out_proj_ref(o, w[torch.from_numpy(cols)])
    _check(u[:, torch.from_numpy(cols).to(DEV)], U, f"T={T} full width, splits={_splits(T, h, n)}")


def test_outproj_deterministic_and_workspace_reused():
    o, w = _inputs(64, 32, 1024, seed=3)
    od, wd = o.to(DEV), w.to(DEV)
    a = outproj(od, wd)
    b = outproj(od, wd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
