"""Exact scaled dot-product attention on MI355X (gfx950).

A thin binding over libattn.so (the C ABI in include/attn.h).  Every step of the
computation runs in the library's HIP kernels; this module only checks tensor
metadata and passes device pointers, sizes and the current HIP stream.  PyTorch
provides device memory and streams.

Functions carry the names of the C entry points:

    attn_fwd(q, k, v, scale=None, causal=False, o=None, lse=None, return_lse=True)
    attn_fwd_fp8(q, k, v, scale=None, v_scale=1.0, causal=False, o=None, lse=None, return_lse=True)
    attn_decode(q, k_cache, v_cache, seq_lens, scale=None, o=None, lse=None,
                workspace=None, return_lse=True)
    attn_decode_split(q, k_cache, v_cache, seq_lens, keys_per_split, scale=None, o=None,
                      lse=None, workspace=None, return_lse=True)
    attn_decode_noalloc(q, k_cache, v_cache, seq_lens, o, lse=None, scale=None)
    attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, o=None,
                      lse=None, workspace=None, keys_per_split=0, return_lse=True)
    attn_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, d)
    attn_decode_split_workspace_bytes(B, Hq, Hkv, max_seq_len, d, keys_per_split)
    attn_bwd(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
             workspace=None)
    attn_bwd_workspace_bytes(B, Hq, Nq)
    attn_status_str(status)

There is no fallback: if libattn.so is missing or a call fails, an exception is
raised.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_LAUNCH,
    ATTN_ERR_UNSUPPORTED,
    ATTN_ERR_WORKSPACE,
    ATTN_F32,
    ATTN_OK,
    AttnError,
    attn_bwd,
    attn_bwd_workspace_bytes,
    attn_decode,
    attn_decode_noalloc,
    attn_decode_paged,
    attn_decode_split,
    attn_decode_split_workspace_bytes,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_fp8,
    attn_status_str,
    lib,
    lib_path,
)

__all__ = [
    "attn_fwd",
    "attn_fwd_fp8",
    "attn_decode",
    "attn_decode_noalloc",
    "attn_decode_paged",
    "attn_decode_split",
    "attn_decode_workspace_bytes",
    "attn_decode_split_workspace_bytes",
    "attn_bwd",
    "attn_bwd_workspace_bytes",
    "attn_status_str",
    "AttnError",
]
