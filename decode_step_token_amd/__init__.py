"""MI355X-native per-step batched sampler (HIP kernels for gfx950 behind a C ABI).

The sampler turns a decode step's [B, V] logits plus per-request
temperature / top_k / top_p into one int32 token per request, writes it
into the on-device token pool and copies it asynchronously to pinned host
memory; the next step's input ids are gathered from the same pool, the
sampling parameters are prepared from host arrays and a step's new KV pages
are written into the page table.  See ``include/sampler.h`` for the C ABI; this package is its
ctypes binding.
"""
from ._binding import (EXPORTS, LIB_PATH, SAMPLER_BF16, SAMPLER_CHECK_DUPLICATE_ROWS, SAMPLER_DEBUG_TOPK,
                       SAMPLER_F32, Sampler,
                       SamplerArgs, SamplerDebug, SamplerError, gather_tokens, load, sample_batch,
                       sample_batch_static, sampler_check, sampler_create, sampler_destroy, sampler_prepare,
                       sampler_query, sampler_set_checks, sampler_strerror, sampler_wait, write_page_table,
                       write_tokens)

__all__ = [
    "EXPORTS", "LIB_PATH", "SAMPLER_BF16", "SAMPLER_CHECK_DUPLICATE_ROWS", "SAMPLER_DEBUG_TOPK", "SAMPLER_F32", "Sampler",
    "SamplerArgs", "SamplerDebug", "SamplerError", "gather_tokens", "load", "sample_batch",
    "sample_batch_static", "sampler_check", "sampler_create", "sampler_destroy", "sampler_prepare", "sampler_query",
    "sampler_set_checks", "sampler_strerror", "sampler_wait", "write_page_table", "write_tokens",
]
