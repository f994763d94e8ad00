"""Exact causal GQA attention for MI355X (gfx950): prefill and its backward,
paged decode (also for absorbed multi-head latent attention), chunked prefill
over a paged cache, and the KV append that feeds it.

The computation lives in the HIP library libattn.so (C ABI in include/attn.h);
this package only marshals torch GPU tensors into those calls. Nothing here
computes attention on the CPU.
"""
from .binding import (  # noqa: F401
    AttnError, AttnLibraryMissing, AttnVariant, LIB_PATH, attn_backward, attn_backward_workspace_size,
    attn_decode, attn_decode_ex, attn_decode_mla, attn_decode_noalloc, attn_decode_mla_num_splits, attn_decode_mla_workspace_size,
    attn_decode_num_splits,
    attn_decode_workspace_size, attn_gather_pages, attn_kv_append, attn_prefill, attn_prefill_ex,
    attn_prefill_paged, attn_status_string, lib,
)
