"""Float64 CPU oracle for causal prefill self-attention + KV-cache image.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``prefill_self_attention_amd``) never imports this package, and this package
imports nothing from it: the two share only the seeded input generators.

The arithmetic lives in ``oracle.c`` (plain C, float64, OpenMP over
(sequence, head)); this module only marshals numpy arrays into it.  See the
header of ``oracle.c`` for the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.oracle_prefill_varlen.argtypes = [p, p, p, p, i32, i32, i32, i32, ctypes.c_float,
                                          p, p, p, p]
    lib.oracle_prefill_varlen.restype = ctypes.c_int
    lib.oracle_prefill_chunked.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p,
                                           ctypes.c_float, p, p, p, p]
    lib.oracle_prefill_chunked.restype = ctypes.c_int
    lib.oracle_prefill_rows.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, p, p,
                                        ctypes.c_float, p, ctypes.c_int64, p]
    lib.oracle_prefill_rows.restype = ctypes.c_int
    lib.oracle_cache_image.argtypes = [p, p, p, i32, i32, i32, i32, p, p, p]
    lib.oracle_cache_image.restype = ctypes.c_int
    lib.oracle_prefill_chunked_paged.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p, i32, p,
                                                 ctypes.c_float, p, p, p]
    lib.oracle_prefill_chunked_paged.restype = ctypes.c_int
    lib.oracle_quantize_rows_int8.argtypes = [p, ctypes.c_int64, i32, p, p]
    lib.oracle_quantize_rows_int8.restype = ctypes.c_int
    lib.oracle_quantize_rows_fp8.argtypes = [p, ctypes.c_int64, i32, p, p]
    lib.oracle_quantize_rows_fp8.restype = ctypes.c_int
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a) -> np.ndarray:
    """bf16 data as a C-contiguous uint16 array of raw bits."""
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch  # local: only when handed torch tensors
        a = a.detach().cpu().contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bits as uint16/int16 or a torch.bfloat16 tensor")
    return a


def _i32(a) -> np.ndarray:
    if hasattr(a, "cpu"):
        a = a.cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _heads(q, k, v):
    """(H, HK): query heads and K/V heads; H must be a multiple of HK [P5 §2.4]."""
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape:
        raise ValueError("q [N, H, D], k and v [N, HK, D] expected")
    N, H, D = q.shape
    if k.shape[0] != N or k.shape[2] != D or H % k.shape[1] != 0:
        raise ValueError("k / v must be [N, HK, D] with HK dividing H")
    return H, k.shape[1]


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("%s: oracle rejected the metadata (code %d)" % (what, rc))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def prefill_varlen(q, k, v, cu_seqlens, scale, k_cache=None, v_cache=None,
                   want_probs=False):
    """Varlen causal prefill.

    q: bf16 [N, H, D]; k, v: bf16 [N, HK, D] with HK dividing H (HK < H:
    grouped K/V heads, query head h reads K/V head h // (H // HK)); uint16
    bits or torch.bfloat16.
    cu_seqlens: int [B + 1].  scale: the float32 value the GPU receives.
    k_cache, v_cache: optional flat bf16 buffers (>= N*H*D elements) holding
    the caller's contents; copies receive the cache image and are returned.
    Returns (out float64 [N,H,D], k_cache_image, v_cache_image, probs).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu = _i32(cu_seqlens)
    N, H, D = q.shape
    _, HK = _heads(q, k, v)
    B = cu.shape[0] - 1
    if cu[-1] != N:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    out = np.zeros((N, H, D), dtype=np.float64)
    kc = vc = None
    if k_cache is not None:
        kc = _u16(k_cache).copy()
        vc = _u16(v_cache).copy()
    probs = None
    if want_probs:
        n = int(cu[1] - cu[0]) if B == 1 else 0
        probs = np.zeros((H, n, n), dtype=np.float64)
    rc = _load().oracle_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu), B, H, HK, D, ctypes.c_float(scale),
        _ptr(out), _ptr(kc) if kc is not None else None,
        _ptr(vc) if vc is not None else None,
        _ptr(probs) if probs is not None else None)
    _check(rc, "prefill_varlen")
    return out, kc, vc, probs


def prefill_chunked(q, k, v, cu_seqlens, prefix_lens, k_cache, v_cache, scale,
                    want_probs=False):
    """Chunked prefill with a cached prefix per sequence.

    k_cache, v_cache: bf16 [B, HK, cap, D] holding the prefix; copies receive
    the image with the new tokens appended and are returned.
    Returns (out float64 [N,H,D], k_cache_image, v_cache_image, probs).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu = _i32(cu_seqlens)
    pre = _i32(prefix_lens)
    kc = _u16(k_cache).copy()
    vc = _u16(v_cache).copy()
    N, H, D = q.shape
    _, HK = _heads(q, k, v)
    B = cu.shape[0] - 1
    cap = kc.shape[2]
    if kc.shape != (B, HK, cap, D) or vc.shape != kc.shape:
        raise ValueError("cache must be [B, HK, cap, D]")
    out = np.zeros((N, H, D), dtype=np.float64)
    probs = None
    if want_probs:
        n = int(cu[1] - cu[0]) if B == 1 else 0
        probs = np.zeros((H, n, int(pre[0]) + n if B == 1 else 0), dtype=np.float64)
    rc = _load().oracle_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu), B, H, HK, D, cap, _ptr(pre),
        ctypes.c_float(scale), _ptr(out), _ptr(kc), _ptr(vc),
        _ptr(probs) if probs is not None else None)
    _check(rc, "prefill_chunked")
    return out, kc, vc, probs


def prefill_rows(q, k, v, cu_seqlens, scale, rows, prefix_lens=None,
                 k_cache=None, v_cache=None):
    """Outputs for the listed token indices only (all heads): float64 [len(rows), H, D].

    For chunked problems pass prefix_lens and the cache *before* the call.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu = _i32(cu_seqlens)
    N, H, D = q.shape
    _, HK = _heads(q, k, v)
    B = cu.shape[0] - 1
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((rows.shape[0], H, D), dtype=np.float64)
    pre = kc = vc = None
    cap = 0
    if prefix_lens is not None:
        pre = _i32(prefix_lens)
        kc = _u16(k_cache)
        vc = _u16(v_cache)
        cap = kc.shape[2]
    rc = _load().oracle_prefill_rows(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu), B, H, HK, D, cap,
        _ptr(pre) if pre is not None else None,
        _ptr(kc) if kc is not None else None,
        _ptr(vc) if vc is not None else None,
        ctypes.c_float(scale), _ptr(rows), rows.shape[0], _ptr(out))
    _check(rc, "prefill_rows")
    return out


def cache_image(k, v, cu_seqlens, k_cache, v_cache, prefix_lens=None):
    """The cache image only (no attention): copies of k_cache / v_cache with
    the new tokens' K/V placed.  Varlen layout if prefix_lens is None (flat
    buffers of >= N*HK*D elements), else chunked [B, HK, cap, D]; HK is k's
    head count."""
    k, v = _u16(k), _u16(v)
    cu = _i32(cu_seqlens)
    N, H, D = k.shape
    B = cu.shape[0] - 1
    kc = _u16(k_cache).copy()
    vc = _u16(v_cache).copy()
    pre = None
    cap = 0
    if prefix_lens is not None:
        pre = _i32(prefix_lens)
        cap = kc.shape[2]
        if kc.shape != (B, H, cap, D) or vc.shape != kc.shape:
            raise ValueError("cache must be [B, H, cap, D]")
    elif kc.size < N * H * D or vc.size < N * H * D:
        raise ValueError("varlen cache needs N*H*D elements")
    rc = _load().oracle_cache_image(_ptr(k), _ptr(v), _ptr(cu), B, H, D, cap,
                                    _ptr(pre) if pre is not None else None,
                                    _ptr(kc), _ptr(vc))
    _check(rc, "cache_image")
    return kc, vc


def quantize_rows_int8(x):
    """INT8 codes and float32 scales of bf16 rows (the last axis is one row):
    symmetric, one scale per row, scale = amax/127, code = rint(x * 127/amax)
    in float32 (see oracle.c).  Returns (codes int8 x.shape, scales float32
    x.shape[:-1])."""
    a = _u16(x)
    d = a.shape[-1]
    rows = a.size // d if d else 0
    codes = np.zeros(a.shape, np.int8)
    scales = np.zeros(a.shape[:-1], np.float32)
    rc = _load().oracle_quantize_rows_int8(_ptr(a), rows, d, _ptr(codes), _ptr(scales))
    _check(rc, "quantize_rows_int8")
    return codes, scales


def cache_image_int8(k, v, cu_seqlens):
    """INT8 varlen cache image: the bf16 varlen image of cache_image (sequence
    b's [HK, len_b, D] block at row cu[b]*HK) with every (token, K/V head) row
    quantised by quantize_rows_int8.  Returns (k_codes, k_scales, v_codes,
    v_scales) as flat arrays of N*HK*D int8 and N*HK float32."""
    kk = _u16(k)
    N, HK, D = kk.shape
    z = np.zeros(N * HK * D, np.uint16)
    kimg, vimg = cache_image(k, v, cu_seqlens, z, z)
    kq, ks = quantize_rows_int8(kimg.reshape(N * HK, D))
    vq, vs = quantize_rows_int8(vimg.reshape(N * HK, D))
    return kq.reshape(-1), ks.reshape(-1), vq.reshape(-1), vs.reshape(-1)


def e4m3_encode(x):
    """The E4M3 code of a float32 value, round to nearest, ties to even (see oracle.c)."""
    return int(_load().oracle_e4m3_encode(float(np.float32(x))))


def e4m3_decode(code):
    """The value an E4M3 code stands for (NaN for S.1111.111)."""
    return float(_load().oracle_e4m3_decode(int(code) & 0xFF))


def quantize_rows_fp8(x):
    """FP8 (E4M3) codes and float32 scales of bf16 rows (the last axis is one
    row): symmetric, one scale per row, scale = amax/448, code =
    E4M3(x * 448/amax) in float32 (see oracle.c).  Returns (codes uint8
    x.shape, scales float32 x.shape[:-1])."""
    a = _u16(x)
    d = a.shape[-1]
    rows = a.size // d if d else 0
    codes = np.zeros(a.shape, np.uint8)
    scales = np.zeros(a.shape[:-1], np.float32)
    rc = _load().oracle_quantize_rows_fp8(_ptr(a), rows, d, _ptr(codes), _ptr(scales))
    _check(rc, "quantize_rows_fp8")
    return codes, scales


def cache_image_fp8(k, v, cu_seqlens):
    """FP8 varlen cache image, laid out as cache_image_int8.  Returns
    (k_codes, k_scales, v_codes, v_scales): N*HK*D uint8 and N*HK float32."""
    kk = _u16(k)
    N, HK, D = kk.shape
    z = np.zeros(N * HK * D, np.uint16)
    kimg, vimg = cache_image(k, v, cu_seqlens, z, z)
    kq, ks = quantize_rows_fp8(kimg.reshape(N * HK, D))
    vq, vs = quantize_rows_fp8(vimg.reshape(N * HK, D))
    return kq.reshape(-1), ks.reshape(-1), vq.reshape(-1), vs.reshape(-1)


def prefill_chunked_paged(q, k, v, cu_seqlens, prefix_lens, k_cache, v_cache, block_table, scale):
    """Chunked prefill over a paged cache (see oracle.c): k_cache / v_cache are
    [num_blocks, HK, 16, D] bf16, block_table [B, max_blocks_per_seq] int32.
    Returns (out float64 [N, H, D], k_cache image, v_cache image)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu = _i32(cu_seqlens)
    pre = _i32(prefix_lens)
    bt = _i32(block_table)
    kc = _u16(k_cache).copy()
    vc = _u16(v_cache).copy()
    N, H, D = q.shape
    HK = k.shape[1]
    B = cu.shape[0] - 1
    nb = kc.shape[0]
    if kc.shape != (nb, HK, 16, D) or vc.shape != kc.shape:
        raise ValueError("paged cache must be [num_blocks, HK, 16, D]")
    if bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("block table must be [B, max_blocks_per_seq]")
    out = np.zeros((N, H, D), np.float64)
    rc = _load().oracle_prefill_chunked_paged(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu), B, H, HK, D, nb, _ptr(bt), bt.shape[1], _ptr(pre),
        ctypes.c_float(scale), _ptr(out), _ptr(kc), _ptr(vc))
    _check(rc, "prefill_chunked_paged")
    return out, kc, vc
