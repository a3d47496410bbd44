"""Thin ctypes binding over libprefill_attn.so (include/prefill_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprefill_attn.so")

PA_OK = 0
_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libprefill_attn.so is not built (%s); run `python -m prefill_self_attention_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.prefill_attn_varlen.argtypes = [p, p, p, p, i32, i32, i32, i32, p, p, p,
                                        ctypes.c_float, p]
    lib.prefill_attn_varlen.restype = ctypes.c_int
    lib.prefill_attn_chunked.argtypes = [p, p, p, p, i32, i32, i32, i32, p, p, i32, p,
                                         ctypes.c_float, p, p]
    lib.prefill_attn_chunked.restype = ctypes.c_int
    lib.prefill_attn_varlen_gqa.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, p, p,
                                            ctypes.c_float, p]
    lib.prefill_attn_varlen_gqa.restype = ctypes.c_int
    lib.prefill_attn_chunked_gqa.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, p, i32, p,
                                             ctypes.c_float, p, p]
    lib.prefill_attn_chunked_gqa.restype = ctypes.c_int
    lib.prefill_attn_varlen_int8.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, p, p, p, p,
                                             ctypes.c_float, p]
    lib.prefill_attn_varlen_int8.restype = ctypes.c_int
    lib.prefill_attn_varlen_fp8.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, p, p, p, p,
                                             ctypes.c_float, p]
    lib.prefill_attn_varlen_fp8.restype = ctypes.c_int
    lib.prefill_attn_chunked_splitkv.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, p, p,
                                                 i32, p, ctypes.c_float, p, p, p, ctypes.c_size_t]
    lib.prefill_attn_chunked_splitkv.restype = ctypes.c_int
    lib.prefill_attn_chunked_splitkv_paged.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32,
                                                       p, p, i32, p, i32, p, ctypes.c_float, p,
                                                       p, p, ctypes.c_size_t]
    lib.prefill_attn_chunked_splitkv_paged.restype = ctypes.c_int
    lib.prefill_attn_splitkv_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.prefill_attn_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.prefill_attn_chunked_splitkv_noalloc.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32,
                                                         p, p, i32, p, ctypes.c_float, p, p]
    lib.prefill_attn_chunked_splitkv_noalloc.restype = ctypes.c_int
    lib.prefill_attn_splitkv_noalloc_limit.argtypes = []
    lib.prefill_attn_splitkv_noalloc_limit.restype = ctypes.c_size_t
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_set_check_mode.argtypes = [ctypes.c_int]
    lib.pa_set_check_mode.restype = ctypes.c_int
    lib.pa_last_hip_error.argtypes = []
    lib.pa_last_hip_error.restype = ctypes.c_int
    _lib = lib
    return lib


def pa_status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def pa_set_check_mode(on: bool) -> bool:
    return bool(load().pa_set_check_mode(1 if on else 0))


def pa_last_hip_error() -> int:
    return int(load().pa_last_hip_error())


class PrefillAttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = int(status)
        msg = pa_status_string(status)
        if status == 9:
            msg += " (hipError_t %d)" % pa_last_hip_error()
        super().__init__(msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check_tensor(name, t, dtype):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)


def _max_seqlen(cu_seqlens) -> int:
    """max(cu[b+1]-cu[b]) from a host copy (synchronises the stream)."""
    c = cu_seqlens.cpu().tolist()
    return max([c[i + 1] - c[i] for i in range(len(c) - 1)] or [0])


def _heads(q, k, v):
    """(H, HK, D): k and v may carry fewer heads than q (grouped K/V heads)."""
    if q.dim() != 3 or k.dim() != 3 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q must be [N, H, D] and k, v [N, HK, D]")
    N, H, D = q.shape
    if k.shape[0] != N or k.shape[2] != D:
        raise ValueError("k/v must be [N, HK, D] with q's N and D")
    return H, k.shape[1], D


def prefill_attn_varlen(q, k, v, cu_seqlens, k_cache, v_cache, out, scale=None,
                        max_seqlen=None, stream=None):
    """Varlen causal prefill + KV-cache write (see prefill_attn.h).

    q, out: bf16 [N, H, D] device tensors; k, v: bf16 [N, HK, D] with HK
    dividing H (HK < H: grouped K/V heads, prefill_attn_varlen_gqa);
    cu_seqlens: int32 [B + 1] device; k_cache, v_cache: bf16 device tensors of
    N*HK*D elements (sequence b's [HK, len_b, D] block starts at element
    cu[b]*HK*D).  scale defaults to 1/sqrt(D).  max_seqlen: host int; computed
    from cu_seqlens (a sync) if omitted.  Returns out.
    """
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("out", out)):
        _check_tensor(n, t, torch.bfloat16)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32)
    H, HK, D = _heads(q, k, v)
    B = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen is None:
        max_seqlen = _max_seqlen(cu_seqlens)
    st = load().prefill_attn_varlen_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, int(max_seqlen), H, HK, D,
        _ptr(k_cache), _ptr(v_cache), _ptr(out), ctypes.c_float(scale), _stream(stream))
    if st != PA_OK:
        raise PrefillAttnError(st)
    return out


def prefill_attn_chunked(q, k, v, cu_seqlens, k_cache, v_cache, out, prefix_lens,
                         scale=None, max_seqlen=None, stream=None):
    """Chunked prefill: new tokens attend to a cached prefix and to each other.

    k_cache, v_cache: bf16 [B, HK, cap, D] device; prefix_lens: int32 [B]
    device.  New tokens' K/V are written at positions prefix_b .. prefix_b +
    len_b - 1.  Other arguments as for prefill_attn_varlen.  Returns out.
    """
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("out", out)):
        _check_tensor(n, t, torch.bfloat16)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32)
    _check_tensor("prefix_lens", prefix_lens, torch.int32)
    H, HK, D = _heads(q, k, v)
    B = cu_seqlens.shape[0] - 1
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[1] != HK or \
            k_cache.shape[3] != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [B, HK, cap, D]")
    cap = k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen is None:
        max_seqlen = _max_seqlen(cu_seqlens)
    st = load().prefill_attn_chunked_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, int(max_seqlen), H, HK, D,
        _ptr(k_cache), _ptr(v_cache), int(cap), _ptr(out), ctypes.c_float(scale),
        _stream(stream), _ptr(prefix_lens))
    if st != PA_OK:
        raise PrefillAttnError(st)
    return out


def splitkv_workspace_size(num_seqs: int, num_tokens: int, num_heads: int, head_dim: int,
                           cache_capacity: int) -> int:
    """Bytes of device workspace prefill_attn_chunked_splitkv needs (0: invalid sizes)."""
    return int(load().prefill_attn_splitkv_workspace_size(
        int(num_seqs), int(num_tokens), int(num_heads), int(head_dim), int(cache_capacity)))


def prefill_attn_chunked_splitkv(q, k, v, cu_seqlens, k_cache, v_cache, out, prefix_lens,
                                 scale=None, max_seqlen=None, stream=None, workspace=None):
    """Chunked prefill with split key ranges and a log-sum-exp merge.

    Same arguments and result as prefill_attn_chunked (up to rounding order).
    workspace: a uint8 device tensor of at least splitkv_workspace_size(...)
    bytes; allocated here through torch when omitted.  Returns out.
    """
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("out", out)):
        _check_tensor(n, t, torch.bfloat16)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32)
    _check_tensor("prefix_lens", prefix_lens, torch.int32)
    H, HK, D = _heads(q, k, v)
    N = q.shape[0]
    B = cu_seqlens.shape[0] - 1
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[1] != HK or \
            k_cache.shape[3] != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [B, HK, cap, D]")
    cap = k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen is None:
        max_seqlen = _max_seqlen(cu_seqlens)
    need = splitkv_workspace_size(B, N, H, D, cap)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_tensor("workspace", workspace, torch.uint8)
    st = load().prefill_attn_chunked_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, int(max_seqlen), N, H, HK, D,
        _ptr(k_cache), _ptr(v_cache), int(cap), _ptr(out), ctypes.c_float(scale),
        _stream(stream), _ptr(prefix_lens), _ptr(workspace), workspace.numel())
    if st != PA_OK:
        raise PrefillAttnError(st)
    return out


def splitkv_noalloc_limit() -> int:
    """Bytes of the per-GPU array prefill_attn_chunked_splitkv_noalloc uses."""
    return int(load().prefill_attn_splitkv_noalloc_limit())


def prefill_attn_chunked_splitkv_noalloc(q, k, v, cu_seqlens, k_cache, v_cache, out, prefix_lens,
                                         scale=None, max_seqlen=None, stream=None):
    """prefill_attn_chunked_splitkv with the library's fixed per-GPU scratch
    array in place of a workspace: allocates nothing.  Calls that overlap in
    time on one GPU race on the array.  Returns out."""
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("out", out)):
        _check_tensor(n, t, torch.bfloat16)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32)
    _check_tensor("prefix_lens", prefix_lens, torch.int32)
    H, HK, D = _heads(q, k, v)
    N = q.shape[0]
    B = cu_seqlens.shape[0] - 1
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[1] != HK or \
            k_cache.shape[3] != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [B, HK, cap, D]")
    cap = k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen is None:
        max_seqlen = _max_seqlen(cu_seqlens)
    st = load().prefill_attn_chunked_splitkv_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, int(max_seqlen), N, H, HK, D,
        _ptr(k_cache), _ptr(v_cache), int(cap), _ptr(out), ctypes.c_float(scale),
        _stream(stream), _ptr(prefix_lens))
    if st != PA_OK:
        raise PrefillAttnError(st)
    return out


def _varlen_quant(q, k, v, cu_seqlens, k_cache, v_cache, k_scale, v_scale, out, scale, max_seqlen,
                  stream, code_dtype, entry, what):
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_tensor(n, t, torch.bfloat16)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, t, code_dtype)
    for n, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(n, t, torch.float32)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32)
    H, HK, D = _heads(q, k, v)
    N = q.shape[0]
    if k_cache.numel() < N * HK * D or v_cache.numel() < N * HK * D or \
            k_scale.numel() < N * HK or v_scale.numel() < N * HK:
        raise ValueError("%s cache needs N*HK*D codes and N*HK scales per matrix" % what)
    B = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen is None:
        max_seqlen = _max_seqlen(cu_seqlens)
    st = getattr(load(), entry)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, int(max_seqlen), H, HK, D,
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        ctypes.c_float(scale), _stream(stream))
    if st != PA_OK:
        raise PrefillAttnError(st)
    return out


def prefill_attn_varlen_int8(q, k, v, cu_seqlens, k_cache, v_cache, k_scale, v_scale, out,
                             scale=None, max_seqlen=None, stream=None):
    """Varlen causal prefill writing an INT8 KV cache (see prefill_attn.h).

    Attention as prefill_attn_varlen; k_cache, v_cache: int8 device tensors of
    N*HK*D elements (varlen layout), k_scale, v_scale: float32 device tensors
    of N*HK elements (one scale per token and K/V head).  Returns out.
    """
    import torch
    return _varlen_quant(q, k, v, cu_seqlens, k_cache, v_cache, k_scale, v_scale, out, scale, max_seqlen,
                         stream, torch.int8, "prefill_attn_varlen_int8", "INT8")


def prefill_attn_varlen_fp8(q, k, v, cu_seqlens, k_cache, v_cache, k_scale, v_scale, out,
                            scale=None, max_seqlen=None, stream=None):
    """Varlen causal prefill writing an FP8 (E4M3) KV cache (see prefill_attn.h).

    As prefill_attn_varlen_int8 with uint8 code tensors holding E4M3 bytes.
    Returns out.
    """
    import torch
    return _varlen_quant(q, k, v, cu_seqlens, k_cache, v_cache, k_scale, v_scale, out, scale, max_seqlen,
                         stream, torch.uint8, "prefill_attn_varlen_fp8", "FP8")


def prefill_attn_chunked_splitkv_paged(q, k, v, cu_seqlens, k_cache, v_cache, block_table, out,
                                       prefix_lens, scale=None, max_seqlen=None, stream=None,
                                       workspace=None):
    """Split-KV chunked prefill over a paged cache (see prefill_attn.h).

    k_cache, v_cache: bf16 [num_blocks, HK, 16, D] device; block_table: int32
    [B, max_blocks_per_seq] device.  Other arguments as
    prefill_attn_chunked_splitkv.  Returns out.
    """
    import torch
    for n, t in (("q", q), ("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("out", out)):
        _check_tensor(n, t, torch.bfloat16)
    for n, t in (("cu_seqlens", cu_seqlens), ("prefix_lens", prefix_lens),
                 ("block_table", block_table)):
        _check_tensor(n, t, torch.int32)
    H, HK, D = _heads(q, k, v)
    N = q.shape[0]
    B = cu_seqlens.shape[0] - 1
    if k_cache.dim() != 4 or k_cache.shape[1] != HK or k_cache.shape[2] != 16 or \
            k_cache.shape[3] != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks, HK, 16, D]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    nb, mb = k_cache.shape[0], block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen is None:
        max_seqlen = _max_seqlen(cu_seqlens)
    need = splitkv_workspace_size(B, N, H, D, 16 * mb)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_tensor("workspace", workspace, torch.uint8)
    st = load().prefill_attn_chunked_splitkv_paged(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, int(max_seqlen), N, H, HK, D,
        _ptr(k_cache), _ptr(v_cache), int(nb), _ptr(block_table), int(mb), _ptr(out),
        ctypes.c_float(scale), _stream(stream), _ptr(prefix_lens), _ptr(workspace),
        workspace.numel())
    if st != PA_OK:
        raise PrefillAttnError(st)
    return out
