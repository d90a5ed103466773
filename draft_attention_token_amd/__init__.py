"""MI355X-native token-importance path of Speculative Prefill.

The work runs in ``libspecprefill.so`` (hand-written HIP for gfx950, C ABI in
``include/specprefill.h``); :mod:`draft_attention_token_amd.specprefill` is
the thin ctypes binding.
"""
from .specprefill import (  # noqa: F401
    Batch, Pipeline, SpError, lib, sp_gather_kept, sp_pool_chunk, sp_score_attention,
    sp_select_chunks, status_string,
)
