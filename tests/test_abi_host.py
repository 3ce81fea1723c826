"""The C-ABI library on the host: it loads, exports every entry point the
header declares, and rejects invalid calls before touching the device (so
these run without a GPU)."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _lib():
    from paged_mla_decode_03_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from paged_mla_decode_03_amd.build import build
        build()
    return binding.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(mla_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"mla_get_metadata", "mla_decode_paged", "mla_num_workers", "mla_workspace_bytes",
            "mla_status_string", "mla_decode_splitkv", "mla_decode_splitkv_timed", "mla_combine_splits",
            "mla_sched_fixed_overhead", "mla_kvcache_append", "mla_absorb_q",
            "mla_absorb_o", "mla_check_inputs", "mla_set_debug_checks"} <= names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in the header but not exported"


def test_single_hip_runtime_in_process():
    _lib()
    maps = open("/proc/self/maps").read().splitlines()
    runtimes = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(runtimes) == 1, runtimes


def test_status_strings():
    lib = _lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.mla_status_string(code) != b"unknown status"
    assert b"WORKSPACE" in lib.mla_status_string(-3)
    assert b"BAD_INPUT" in lib.mla_status_string(-6)


def test_workspace_bytes():
    lib = _lib()
    got = lib.mla_workspace_bytes(64, 1, 128, 1, 512, 256)
    a256 = lambda x: (x + 255) // 256 * 256
    slots, rows = 256 + 64, 128
    assert got == a256(slots * rows * 512 * 4) + a256(slots * rows * 4)
    assert lib.mla_workspace_bytes(0, 1, 128, 1, 512, 256) == 0
    assert lib.mla_workspace_bytes(2, 1, 128, 3, 512, 256) == 0     # h_q % h_kv != 0
    assert lib.mla_workspace_bytes(2, 1, 128, 1, 256, 256) == 0     # dv != 512


def test_fixed_overhead_matches_reference_rule():
    from oracle.sched_ref import FIXED_OVERHEAD_PAGES
    assert _lib().mla_sched_fixed_overhead() == FIXED_OVERHEAD_PAGES


FAKE = 0x10000   # 64 KB-aligned, never dereferenced: every call below fails validation first


def _decode(lib, entry="mla_decode_paged", **kw):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, max_pages=4, num_pages=8, seqlens=FAKE, batch=2, s_q=1, h_q=16,
                h_kv=1, d_qk=576, dv=512, meta=FAKE, ns=FAKE, W=256, causal=0, scale=0.0, o=FAKE, lse=FAKE,
                ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return getattr(lib, entry)(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(kv=None), -1), (dict(o=None), -1), (dict(ws=None), -1),
    (dict(batch=0), -1), (dict(s_q=0), -1), (dict(h_q=16, h_kv=3), -1), (dict(max_pages=0), -1),
    (dict(causal=2), -1),
    (dict(d_qk=512), -2), (dict(dv=576), -2), (dict(q=FAKE + 8), -2), (dict(o=FAKE + 4), -2),
    (dict(ws=FAKE + 16), -2),
    (dict(ws_bytes=1024), -3),
    (dict(W=0), -4), (dict(W=5000), -4),
])
@pytest.mark.parametrize("entry", ["mla_decode_paged", "mla_decode_splitkv"])
def test_decode_rejects_invalid_arguments(kw, status, entry):
    assert _decode(_lib(), entry, **kw) == status


def test_timed_decode_rejects_invalid_arguments():
    lib = _lib()
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, max_pages=4, num_pages=8, seqlens=FAKE, batch=2, s_q=1, h_q=16,
                h_kv=1, d_qk=576, dv=512, meta=FAKE, ns=FAKE, W=256, causal=0, scale=0.0, o=FAKE, lse=FAKE,
                ws=FAKE, ws_bytes=1 << 30, stream=None)
    # the same checks as mla_decode_splitkv, then both events are required
    assert lib.mla_decode_splitkv_timed(*args.values(), FAKE, None) == -1
    assert lib.mla_decode_splitkv_timed(*args.values(), None, FAKE) == -1
    args.update(q=None)
    assert lib.mla_decode_splitkv_timed(*args.values(), FAKE, FAKE) == -1
    args.update(q=FAKE, ws_bytes=1024)
    assert lib.mla_decode_splitkv_timed(*args.values(), FAKE, FAKE) == -3


def test_metadata_and_combine_reject_invalid_arguments():
    lib = _lib()
    assert lib.mla_get_metadata(None, 2, 16, 1, 256, FAKE, FAKE, None) == -1
    assert lib.mla_get_metadata(FAKE, 0, 16, 1, 256, FAKE, FAKE, None) == -1
    assert lib.mla_get_metadata(FAKE, 2, 16, 1, 0, FAKE, FAKE, None) == -4
    assert lib.mla_get_metadata(FAKE + 2, 2, 16, 1, 256, FAKE, FAKE, None) == -2
    assert lib.mla_combine_splits(None, 2, 1, 16, 1, 512, 256, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.mla_combine_splits(FAKE, 2, 1, 16, 1, 512, 256, FAKE, FAKE, FAKE, 16, None) == -3
    assert lib.mla_combine_splits(FAKE, 2, 1, 16, 1, 256, 256, FAKE, FAKE, FAKE, 1 << 30, None) == -2
    n = ctypes.c_int(0)
    assert lib.mla_num_workers(0, 0, 1, ctypes.byref(n)) == -1
    assert lib.mla_num_workers(0, 16, 1, None) == -1


def test_append_rejects_invalid_arguments():
    lib = _lib()
    ok = dict(kv_new=FAKE, kv=FAKE, bt=FAKE, max_pages=4, num_pages=8, L=FAKE, batch=2, s_new=1, h_kv=1, d=576,
              bad=None, stream=None)
    for kw, status in [(dict(kv_new=None), -1), (dict(kv=None), -1), (dict(bt=None), -1), (dict(L=None), -1),
                       (dict(batch=0), -1), (dict(s_new=0), -1), (dict(h_kv=0), -1), (dict(max_pages=0), -1),
                       (dict(num_pages=-1), -1), (dict(d=512), -2), (dict(kv_new=FAKE + 8), -2),
                       (dict(kv=FAKE + 8), -2), (dict(bt=FAKE + 2), -2), (dict(bad=FAKE + 2), -2),
                       (dict(batch=1 << 20, s_new=1 << 6), -2), (dict(num_pages=1 << 30), -2)]:
        args = dict(ok, **kw)
        assert lib.mla_kvcache_append(*args.values()) == status, kw


def test_absorb_rejects_invalid_arguments():
    lib = _lib()
    assert lib.mla_absorb_q(None, FAKE, FAKE, FAKE, 4, 128, None) == -1
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, FAKE, 0, 128, None) == -1
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, FAKE, 4, -1, None) == -1
    assert lib.mla_absorb_q(FAKE, FAKE + 8, FAKE, FAKE, 4, 128, None) == -2
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, FAKE, 1 << 20, 128, None) == -2
    assert lib.mla_absorb_o(FAKE, None, FAKE, 4, 128, None) == -1
    assert lib.mla_absorb_o(FAKE, FAKE, FAKE + 2, 4, 128, None) == -2
    assert lib.mla_absorb_o(FAKE, FAKE, FAKE, 4, 0, None) == -1


def test_check_inputs_rejects_invalid_arguments():
    lib = _lib()
    ok = dict(bt=FAKE, max_pages=4, num_pages=8, L=FAKE, batch=2, result=FAKE, stream=None)
    for kw, status in [(dict(bt=None), -1), (dict(L=None), -1), (dict(result=None), -1), (dict(batch=0), -1),
                       (dict(max_pages=0), -1), (dict(num_pages=0), -1), (dict(bt=FAKE + 2), -2),
                       (dict(L=FAKE + 1), -2), (dict(result=FAKE + 2), -2)]:
        args = dict(ok, **kw)
        assert lib.mla_check_inputs(*args.values()) == status, kw


def _cpu_buffers(B, s_q, h_q, W, o_shape=None, lse_shape=None, ws_bytes=None):
    from paged_mla_decode_03_amd import binding
    buf = binding.DecodeBuffers.__new__(binding.DecodeBuffers)
    buf.o = torch.empty(o_shape or (B, s_q, h_q, 512), dtype=torch.bfloat16)
    buf.lse = torch.empty(lse_shape or (B, h_q, s_q), dtype=torch.float32)
    need = binding.workspace_bytes(B, s_q, h_q, 1, 512, W)
    buf.workspace = torch.empty(need if ws_bytes is None else ws_bytes, dtype=torch.uint8)
    return buf


def test_decode_buffers_must_match_the_call():
    """The library writes o and lse for every (b, i, h) of a call, so
    caller-supplied buffers of another shape are refused before any launch."""
    from paged_mla_decode_03_amd import binding
    _lib()
    cpu = torch.device("cpu")
    binding._check_buffers(_cpu_buffers(4, 2, 16, 8), 4, 2, 16, 1, 512, 8, cpu)   # matching: accepted
    for kw in (dict(o_shape=(3, 2, 16, 512)), dict(o_shape=(4, 1, 16, 512)), dict(o_shape=(4, 2, 8, 512)),
               dict(lse_shape=(4, 2, 16)), dict(lse_shape=(4, 16, 1)), dict(ws_bytes=256)):
        with pytest.raises(ValueError):
            binding._check_buffers(_cpu_buffers(4, 2, 16, 8, **kw), 4, 2, 16, 1, 512, 8, cpu)


def test_absorb_outputs_must_match_the_call():
    from paged_mla_decode_03_amd import absorb_o, absorb_q
    _lib()
    qn = torch.zeros((3, 4, 128), dtype=torch.bfloat16)
    qr = torch.zeros((3, 4, 64), dtype=torch.bfloat16)
    w = torch.zeros((4, 512, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        absorb_q(qn, qr, w, out=torch.zeros((2, 4, 576), dtype=torch.bfloat16))
    o = torch.zeros((3, 4, 512), dtype=torch.bfloat16)
    wv = torch.zeros((4, 128, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        absorb_o(o, wv, out=torch.zeros((3, 4, 64), dtype=torch.bfloat16))


def test_pages_calls_reject_invalid_arguments():
    lib = _lib()
    assert lib.mla_pages_init(None, FAKE, 8, None) == -1
    assert lib.mla_pages_init(FAKE, FAKE, 0, None) == -1
    assert lib.mla_pages_init(FAKE + 2, FAKE, 8, None) == -2
    ok = dict(fp=FAKE, st=FAKE, P=8, L=FAKE, B=2, s_new=1, bt=FAKE, mp=4, stream=None)
    for kw, status in [(dict(fp=None), -1), (dict(bt=None), -1), (dict(P=0), -1), (dict(B=0), -1),
                       (dict(s_new=-1), -1), (dict(mp=0), -1), (dict(L=FAKE + 1), -2), (dict(st=FAKE + 2), -2)]:
        args = dict(ok, **kw)
        assert lib.mla_pages_reserve(*args.values()) == status, kw
    ok = dict(fp=FAKE, st=FAKE, P=8, L=FAKE, rel=FAKE, B=2, bt=FAKE, mp=4, stream=None)
    for kw, status in [(dict(rel=None), -1), (dict(B=-1), -1), (dict(rel=FAKE + 1), -2), (dict(bt=FAKE + 2), -2)]:
        args = dict(ok, **kw)
        assert lib.mla_pages_release(*args.values()) == status, kw


def test_outproj_rejects_invalid_arguments():
    lib = _lib()
    assert lib.mla_outproj(None, FAKE, FAKE, 4, 256, 128, FAKE, 1 << 30, None) == -1
    assert lib.mla_outproj(FAKE, FAKE, FAKE, 0, 256, 128, FAKE, 1 << 30, None) == -1
    assert lib.mla_outproj(FAKE, FAKE, FAKE, 4, 200, 128, FAKE, 1 << 30, None) == -2    # k % 128
    assert lib.mla_outproj(FAKE, FAKE, FAKE, 4, 256, 100, FAKE, 1 << 30, None) == -2    # n % 128
    assert lib.mla_outproj(FAKE + 8, FAKE, FAKE, 4, 256, 128, FAKE, 1 << 30, None) == -2


def test_lds_read_rate_rejects_invalid_arguments():
    lib = _lib()
    c = ctypes.c_int
    vp = ctypes.c_void_p
    lib.mla_lds_read_rate.restype = c
    lib.mla_lds_read_rate.argtypes = [c, c, c, c, vp, vp, vp]
    good = vp(4096)   # never dereferenced: every call below fails its argument checks first
    assert lib.mla_lds_read_rate(0, 4, 1, 1, None, good, None) != 0
    assert lib.mla_lds_read_rate(0, 4, 1, 1, good, None, None) != 0
    assert lib.mla_lds_read_rate(4, 4, 1, 1, good, good, None) != 0
    assert lib.mla_lds_read_rate(-1, 4, 1, 1, good, good, None) != 0
    assert lib.mla_lds_read_rate(0, 6, 1, 1, good, good, None) != 0
    assert lib.mla_lds_read_rate(0, 4, 0, 1, good, good, None) != 0
    assert lib.mla_lds_read_rate(0, 4, 1, 0, good, good, None) != 0
    assert lib.mla_lds_read_rate(0, 4, 1, 1, vp(4100), good, None) != 0
