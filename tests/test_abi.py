"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before anything is enqueued (no GPU needed:
none of these calls reaches a HIP runtime call)."""
import ctypes
import math
import os
import re

import pytest

import prefill_self_attention_amd as P
from prefill_self_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return P.load()


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted([
        "prefill_attn_varlen", "prefill_attn_chunked", "prefill_attn_varlen_gqa",
        "prefill_attn_chunked_gqa", "prefill_attn_chunked_splitkv", "prefill_attn_varlen_int8",
        "prefill_attn_varlen_fp8",
        "prefill_attn_chunked_splitkv_paged",
        "prefill_attn_splitkv_workspace_size", "pa_status_string", "pa_set_check_mode",
        "pa_last_hip_error", "prefill_attn_chunked_splitkv_noalloc",
        "prefill_attn_splitkv_noalloc_limit"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in range(12):
        s = P.pa_status_string(code)
        assert s.startswith("PA_")
    assert P.pa_status_string(42) == "unknown pa_status"


def test_check_mode_toggle(lib):
    prev = P.pa_set_check_mode(True)
    assert P.pa_set_check_mode(False) is True
    P.pa_set_check_mode(prev)
    assert P.pa_last_hip_error() == 0


# Fake, never-dereferenced device addresses (16-byte aligned, distinct).
A = [0x10000 * (i + 1) for i in range(10)]


def varlen(lib, q=A[0], k=A[1], v=A[2], cu=A[3], B=1, maxlen=16, H=2, D=64, kc=A[4],
           vc=A[5], out=A[6], scale=0.125):
    return lib.prefill_attn_varlen(q, k, v, cu, B, maxlen, H, D, kc, vc, out,
                                   ctypes.c_float(scale), None)


def chunked(lib, q=A[0], k=A[1], v=A[2], cu=A[3], B=1, maxlen=16, H=2, D=64, kc=A[4],
            vc=A[5], cap=32, out=A[6], scale=0.125, pre=A[7]):
    return lib.prefill_attn_chunked(q, k, v, cu, B, maxlen, H, D, kc, vc, cap, out,
                                    ctypes.c_float(scale), None, pre)


WS = 1 << 40  # a workspace size no test call can exceed


def splitkv(lib, q=A[0], k=A[1], v=A[2], cu=A[3], B=1, maxlen=16, H=2, D=64, kc=A[4],
            vc=A[5], cap=32, out=A[6], scale=0.125, pre=A[7], N=16, HK=None, ws=A[8],
            ws_bytes=WS):
    return lib.prefill_attn_chunked_splitkv(q, k, v, cu, B, maxlen, N, H, H if HK is None else HK,
                                            D, kc, vc, cap, out, ctypes.c_float(scale), None,
                                            pre, ws, ws_bytes)


def varlen_int8(lib, q=A[0], k=A[1], v=A[2], cu=A[3], B=1, maxlen=16, H=2, D=64, kc=A[4],
                vc=A[5], out=A[6], scale=0.125, ks=A[7], vs=A[8], HK=None):
    return lib.prefill_attn_varlen_int8(q, k, v, cu, B, maxlen, H, H if HK is None else HK, D,
                                        kc, vc, ks, vs, out, ctypes.c_float(scale), None)


def varlen_fp8(lib, q=A[0], k=A[1], v=A[2], cu=A[3], B=1, maxlen=16, H=2, D=64, kc=A[4],
               vc=A[5], out=A[6], scale=0.125, ks=A[7], vs=A[8], HK=None):
    return lib.prefill_attn_varlen_fp8(q, k, v, cu, B, maxlen, H, H if HK is None else HK, D,
                                       kc, vc, ks, vs, out, ctypes.c_float(scale), None)


@pytest.mark.parametrize("f", [varlen_int8, varlen_fp8])
def test_quantised_cache_rejections(lib, f):
    assert f(lib, ks=None) == 1
    assert f(lib, vs=None) == 1
    assert f(lib, ks=A[7] + 4) == 5
    assert f(lib, vs=A[6]) == 6     # scale buffer is out
    assert f(lib, ks=A[0]) == 6     # scale buffer is q
    assert f(lib, kc=A[5]) == 6     # both code buffers the same
    assert f(lib, HK=3) == 2
    assert f(lib, D=48) == 3
    assert f(lib, B=0) == 0 and f(lib, maxlen=0) == 0


@pytest.mark.parametrize("f", [varlen, chunked, splitkv, varlen_int8, varlen_fp8])
def test_host_rejections(lib, f):
    assert f(lib, q=None) == 1
    assert f(lib, out=None) == 1
    assert f(lib, cu=None) == 1
    assert f(lib, B=-1) == 2
    assert f(lib, H=0) == 2
    assert f(lib, maxlen=-5) == 2
    assert f(lib, B=70000) == 2
    for d in (0, 16, 48, 96, 256):
        assert f(lib, D=d) == 3
    assert f(lib, scale=math.nan) == 4
    assert f(lib, scale=math.inf) == 4
    assert f(lib, q=A[0] + 2) == 5
    assert f(lib, kc=A[4] + 8) == 5
    assert f(lib, out=A[0]) == 6
    assert f(lib, kc=A[1]) == 6
    assert f(lib, vc=A[4]) == 6


@pytest.mark.parametrize("f", [chunked, splitkv])
def test_chunked_only_rejections(lib, f):
    assert f(lib, pre=None) == 1
    assert f(lib, cap=0) == 2
    assert f(lib, pre=A[6]) == 6


def test_splitkv_rejections(lib):
    assert splitkv(lib, ws=None) == 1
    assert splitkv(lib, ws=A[8] + 4) == 5
    assert splitkv(lib, ws=A[6]) == 6      # workspace is out
    assert splitkv(lib, ws=A[0]) == 6      # workspace is q
    assert splitkv(lib, N=-1) == 2
    assert splitkv(lib, HK=3) == 2
    need = lib.prefill_attn_splitkv_workspace_size(1, 16, 2, 64, 32)
    assert need > 0
    assert splitkv(lib, ws_bytes=need - 1) == 10
    assert P.pa_status_string(10).startswith("PA_ERR_WORKSPACE")
    # a slab row of 2^32 or more elements is refused before anything else is looked at
    assert splitkv(lib, cap=(1 << 25), D=128) == 2
    assert splitkv(lib, cap=(1 << 27), D=32) == 2
    assert splitkv(lib, cap=(1 << 25) - 1, D=128, ws_bytes=0) == 10


def paged(lib, q=A[0], k=A[1], v=A[2], cu=A[3], B=1, maxlen=16, H=2, D=64, kc=A[4],
          vc=A[5], nb=8, bt=A[9], mb=4, out=A[6], scale=0.125, pre=A[7], N=16, HK=None, ws=A[8],
          ws_bytes=WS):
    return lib.prefill_attn_chunked_splitkv_paged(q, k, v, cu, B, maxlen, N, H,
                                                  H if HK is None else HK, D, kc, vc, nb, bt, mb,
                                                  out, ctypes.c_float(scale), None, pre, ws,
                                                  ws_bytes)


def test_paged_rejections(lib):
    assert paged(lib, bt=None) == 1
    assert paged(lib, nb=0) == 2
    assert paged(lib, mb=0) == 2
    assert paged(lib, bt=A[6]) == 6     # table is out
    assert paged(lib, bt=A[8]) == 6     # table is the workspace
    assert paged(lib, ws=None) == 1
    assert paged(lib, pre=None) == 1
    assert paged(lib, q=A[0] + 2) == 5
    assert paged(lib, B=0) == 0 and paged(lib, N=0) == 0


def test_splitkv_workspace_size():
    f = P.splitkv_workspace_size
    assert f(1, 16, 2, 64, 0) == 0 and f(-1, 16, 2, 64, 8) == 0 and f(1, 16, 2, 48, 8) == 0
    # grows with tokens, heads, head size and (up to 64 segments) capacity
    base = f(65, 576, 32, 128, 8192)
    assert f(65, 1152, 32, 128, 8192) > base and f(65, 576, 32, 128, 16384) > base
    assert f(65, 576, 32, 64, 8192) < base
    # segments of 1024 keys: 8192 keys -> 8 segments of fp32 partials per (token, head)
    assert base >= 576 * 32 * 8 * 129 * 4
    # beyond 64 * 1024 keys the segment count stays at 64
    assert f(1, 128, 8, 128, 1 << 20) < 2 * f(1, 128, 8, 128, 1 << 16) + 4096


@pytest.mark.parametrize("f", [varlen, chunked, splitkv])
def test_empty_problem_is_a_no_op(lib, f):
    # nothing is enqueued: these would fault if anything touched the fake pointers
    assert f(lib, B=0) == 0
    assert f(lib, maxlen=0) == 0
    if f is splitkv:
        assert f(lib, N=0) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libprefill_attn.so")
    with pytest.raises(RuntimeError, match="not built"):
        binding.load()


def test_noalloc_limit_and_rejection(lib):
    # the fixed array's size, and a problem whose workspace exceeds it is
    # refused before any HIP call (dummy 16-byte aligned pointers)
    assert P.splitkv_noalloc_limit() == 128 << 20
    need = P.splitkv_workspace_size(1, 1 << 20, 64, 128, 1 << 20)
    assert need > P.splitkv_noalloc_limit()
    d = ctypes.c_void_p(0x10000)
    st = lib.prefill_attn_chunked_splitkv_noalloc(d, d, d, d, 1, 1 << 20, 1 << 20, 64, 64, 128,
                                                  ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000),
                                                  1 << 20, ctypes.c_void_p(0x40000), ctypes.c_float(0.1),
                                                  None, ctypes.c_void_p(0x50000))
    assert st == 11 and P.pa_status_string(st).startswith("PA_ERR_NOALLOC_LIMIT")
