"""MI355X (gfx950) causal varlen / chunked prefill attention with a fused KV-cache write.

The computation lives in HIP kernels behind the C ABI of include/prefill_attn.h
(libprefill_attn.so, built by ``prefill_self_attention_amd.build``); this
package only binds it.  ``inputs`` holds the seeded synthetic workloads.
"""
from .binding import (PrefillAttnError, load, pa_last_hip_error, pa_set_check_mode,
                      pa_status_string, prefill_attn_chunked, prefill_attn_chunked_splitkv,
                      prefill_attn_chunked_splitkv_noalloc, prefill_attn_chunked_splitkv_paged,
                      prefill_attn_varlen, prefill_attn_varlen_fp8, prefill_attn_varlen_int8,
                      splitkv_noalloc_limit, splitkv_workspace_size)

__all__ = ["prefill_attn_varlen", "prefill_attn_varlen_int8", "prefill_attn_varlen_fp8", "prefill_attn_chunked",
           "prefill_attn_chunked_splitkv", "prefill_attn_chunked_splitkv_paged",
           "prefill_attn_chunked_splitkv_noalloc", "splitkv_noalloc_limit",
           "splitkv_workspace_size", "pa_status_string", "pa_set_check_mode",
           "pa_last_hip_error", "PrefillAttnError", "load"]
