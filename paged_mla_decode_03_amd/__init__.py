"""Paged Multi-head Latent Attention decode for AMD MI355X (gfx950).

The work runs in ``libmla_decode.so`` (hand-written HIP kernels behind a C ABI,
``include/mla_decode.h``); ``binding`` marshals torch tensors into it.
"""
from .binding import (DecodeBuffers, PagePool, kvcache_append_fp8, mla_decode_paged_fp8, absorb_o, absorb_q, MlaError, check_inputs, fixed_overhead_pages,
                      get_mla_metadata, kvcache_append, library, mla_combine_splits, mla_decode_paged,
                      mla_decode_splitkv, mla_decode_splitkv_timed, num_workers, outproj, set_debug_checks,
                      workspace_bytes)

__all__ = ["DecodeBuffers", "PagePool", "kvcache_append_fp8", "mla_decode_paged_fp8", "absorb_o", "absorb_q", "MlaError", "check_inputs", "fixed_overhead_pages",
           "get_mla_metadata", "kvcache_append", "library", "mla_combine_splits", "mla_decode_paged",
           "mla_decode_splitkv", "mla_decode_splitkv_timed", "num_workers", "outproj", "set_debug_checks",
           "workspace_bytes"]
