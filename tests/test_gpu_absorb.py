"""The per-head projections around the decode on the GPU against the
oracle's absorb_q_ref / absorb_o_ref (fp64).

Both outputs are rounded once to bf16 after an fp32 sum, so the bar per
element is 2^-8 of its magnitude plus 1e-3 of the output's RMS (fp32
accumulation over K <= 512 terms adds far less)."""
import numpy as np
import pytest
import torch

from oracle.mla_oracle import absorb_o_ref, absorb_q_ref
from paged_mla_decode_03_amd import absorb_o, absorb_q
from tests.gpu_helpers import DEV
from workloads import bf16_normal

pytestmark = pytest.mark.gpu


def _close(got, want):
    g = got.float().cpu().double().numpy()
    bound = 2.0 ** -8 * np.abs(want) + 1e-3 * np.sqrt(np.mean(want ** 2))
    assert np.isfinite(g).all()
    assert (np.abs(g - want) <= bound).all(), float(np.abs(g - want).max())


@pytest.mark.parametrize("tokens,h", [(1, 128), (15, 16), (64, 128), (65, 3), (264, 128), (130, 7), (1000, 5)])
def test_absorb_q_parity(tokens, h):
    rng = np.random.Generator(np.random.PCG64(tokens * 1000 + h))
    print(f"[absorb_q] tokens={tokens} h={h}", flush=True)
    qn, qr = bf16_normal(rng, (tokens, h, 128)), bf16_normal(rng, (tokens, h, 64))
    w = (bf16_normal(rng, (h, 512, 128)).float() / np.sqrt(128)).to(torch.bfloat16)
    got = absorb_q(qn.to(DEV), qr.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    want = absorb_q_ref(qn, qr, w)
    _close(got, want)
    assert torch.equal(got[..., 512:].cpu(), qr)            # the RoPE part is copied bit for bit


@pytest.mark.parametrize("tokens,h", [(1, 128), (15, 16), (64, 128), (65, 3), (264, 128), (130, 7), (1000, 5)])
def test_absorb_o_parity(tokens, h):
    rng = np.random.Generator(np.random.PCG64(tokens * 1000 + h + 7))
    print(f"[absorb_o] tokens={tokens} h={h}", flush=True)
    o = bf16_normal(rng, (tokens, h, 512))
    w = (bf16_normal(rng, (h, 128, 512)).float() / np.sqrt(512)).to(torch.bfloat16)
    got = absorb_o(o.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    _close(got, absorb_o_ref(o, w))


def test_absorb_batched_shape_and_errors():
    """Leading dimensions [B][s_q] are flattened into tokens; wrong shapes and
    dtypes are refused before anything is launched."""
    rng = np.random.Generator(np.random.PCG64(5))
    qn, qr = bf16_normal(rng, (4, 2, 8, 128)), bf16_normal(rng, (4, 2, 8, 64))
    w = (bf16_normal(rng, (8, 512, 128)).float() / np.sqrt(128)).to(torch.bfloat16)
    got = absorb_q(qn.to(DEV), qr.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    assert got.shape == (4, 2, 8, 576)
    _close(got.reshape(8, 8, 576), absorb_q_ref(qn.reshape(8, 8, 128), qr.reshape(8, 8, 64), w))
    with pytest.raises(ValueError):
        absorb_q(qn.to(DEV), qr.to(DEV), w[:, :, :64].contiguous().to(DEV))
    with pytest.raises(TypeError):
        absorb_o(qn.float().to(DEV), w.to(DEV))
