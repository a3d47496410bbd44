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
        "prefill_attn_chunked_gqa", "pa_status_string", "pa_set_check_mode",
        "pa_last_hip_error"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in range(10):
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


@pytest.mark.parametrize("f", [varlen, chunked])
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


def test_chunked_only_rejections(lib):
    assert chunked(lib, pre=None) == 1
    assert chunked(lib, cap=0) == 2
    assert chunked(lib, pre=A[6]) == 6


@pytest.mark.parametrize("f", [varlen, chunked])
def test_empty_problem_is_a_no_op(lib, f):
    # nothing is enqueued: these would fault if anything touched the fake pointers
    assert f(lib, B=0) == 0
    assert f(lib, maxlen=0) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libprefill_attn.so")
    with pytest.raises(RuntimeError, match="not built"):
        binding.load()
