"""GPU test of the no-allocation split-KV call,
prefill_attn_chunked_splitkv_noalloc (C ABI, through ctypes): two calls in a
row on one GPU, the second smaller, each checked against
prefill_attn_chunked_splitkv with a caller workspace on the same inputs
(outputs to the parity bar of tests/gpu_util.py, caches bit for bit; the
two share their kernels, so they also agree bit for bit), and the first call
against the oracle.  The second call finds the first call's contents in the
fixed array, so it also shows that nothing there has to start at zero."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import SENTINEL, assert_close, bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefill_self_attention_amd as P
    return P.load()


def case(seed, lengths, prefix, cap, H, HK, D):
    g = I.generator(seed)
    cu = I.cu_from_lengths(lengths)
    N, B = cu[-1], len(lengths)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    kc0 = I.randn_bf16(g, (B, HK, cap, D))
    vc0 = I.randn_bf16(g, (B, HK, cap, D))
    s = torch.tensor(SENTINEL, dtype=torch.int16).view(torch.bfloat16)
    for b, p in enumerate(prefix):
        kc0[b, :, p:] = s
        vc0[b, :, p:] = s
    return cu, q, k, v, kc0, vc0


def call(lib, fn, cu, prefix, q, k, v, kc, vc, scale, extra):
    N, H, D = q.shape
    HK = k.shape[1]
    B = len(cu) - 1
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    pred = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    args = [ctypes.c_void_p(t.data_ptr()) for t in (qd, kd, vd, cud)]
    args += [B, max(cu[i + 1] - cu[i] for i in range(B)), N, H, HK, D,
             ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()), kc.shape[2],
             ctypes.c_void_p(out.data_ptr()), ctypes.c_float(scale), None,
             ctypes.c_void_p(pred.data_ptr())] + extra
    st = fn(*args)
    torch.cuda.synchronize()
    assert st == 0, st
    return out


@pytest.mark.parametrize("seed, lengths, prefix, cap, H, HK, D", [
    (71, [300, 1, 1, 1], [1500, 700, 2900, 40], 4096, 8, 8, 128),   # larger first
    (72, [90, 1, 1], [200, 33, 1000], 1152, 4, 2, 128),             # then smaller
])
def test_noalloc_matches_workspace_call(lib, seed, lengths, prefix, cap, H, HK, D):
    cu, q, k, v, kc0, vc0 = case(seed, lengths, prefix, cap, H, HK, D)
    scale = 1.0 / math.sqrt(D)
    say("no-alloc case seed=%d lengths=%s prefix=%s cap=%d H=%d HK=%d D=%d" % (seed, lengths, prefix, cap, H, HK, D))
    need = lib.prefill_attn_splitkv_workspace_size(len(lengths), cu[-1], H, D, cap)
    assert 0 < need <= lib.prefill_attn_splitkv_noalloc_limit()
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
    kc_a, vc_a = kc0.cuda(), vc0.cuda()
    out_a = call(lib, lib.prefill_attn_chunked_splitkv, cu, prefix, q, k, v, kc_a, vc_a, scale,
                 [ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need)])
    kc_b, vc_b = kc0.cuda(), vc0.cuda()
    out_b = call(lib, lib.prefill_attn_chunked_splitkv_noalloc, cu, prefix, q, k, v, kc_b, vc_b,
                 scale, [])
    # the no-allocation call against the workspace call
    assert_close(out_b, out_a.float().cpu(), "no-alloc vs workspace call")
    np.testing.assert_array_equal(bits(kc_b), bits(kc_a))
    np.testing.assert_array_equal(bits(vc_b), bits(vc_a))
    # and against the oracle
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, prefix, kc0, vc0, scale)
    assert_close(out_b, ref, "no-alloc vs oracle")
    np.testing.assert_array_equal(bits(kc_b), kimg)
    np.testing.assert_array_equal(bits(vc_b), vimg)
