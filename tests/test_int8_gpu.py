"""GPU parity for the INT8 KV-cache write (prefill_attn_varlen_int8):
attention outputs against the float64 oracle to the parity bar of
tests/gpu_util.py, INT8 codes and float scales bit for bit against
oracle.cache_image_int8 ("大模型推理优化：Prefill、Decode与KV Cache的工程实践"
§4.3: K and V quantised, Q kept; the oracle fixes the per-row symmetric
reading), guard bands around every output untouched."""
import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import assert_close, say

pytestmark = pytest.mark.gpu

GUARD = 4096
BYTE_SENTINEL = 0x5A
F32_SENTINEL = 0x7FC0DEAD  # a float NaN pattern


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefill_self_attention_amd as P
    P.load()
    yield


def P():
    import prefill_self_attention_amd as mod
    return mod


def guarded_i8(n):
    whole = torch.full((n + 2 * GUARD,), BYTE_SENTINEL, dtype=torch.int8, device="cuda")
    return whole[GUARD:GUARD + n], whole


def guarded_f32(n):
    whole = torch.full((n + 2 * GUARD,), F32_SENTINEL, dtype=torch.int32, device="cuda")
    return whole[GUARD:GUARD + n].view(torch.float32), whole


def guards_ok(whole, sentinel):
    a = whole.cpu().numpy()
    return bool(np.all(a[:GUARD] == sentinel) and np.all(a[-GUARD:] == sentinel))


def run_int8(q, k, v, cu, scale):
    N, H, D = q.shape
    HK = k.shape[1]
    kq, kq_w = guarded_i8(N * HK * D)
    vq, vq_w = guarded_i8(N * HK * D)
    ks, ks_w = guarded_f32(N * HK)
    vs, vs_w = guarded_f32(N * HK)
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    P().prefill_attn_varlen_int8(q.cuda(), k.cuda(), v.cuda(),
                                 torch.tensor(cu, dtype=torch.int32, device="cuda"),
                                 kq, vq, ks, vs, out, scale=scale)
    torch.cuda.synchronize()
    assert guards_ok(kq_w, BYTE_SENTINEL) and guards_ok(vq_w, BYTE_SENTINEL)
    assert guards_ok(ks_w, F32_SENTINEL) and guards_ok(vs_w, F32_SENTINEL)
    return out, kq, vq, ks, vs


def check_codes(k, v, cu, kq, vq, ks, vs, what):
    rk, rks, rv, rvs = oracle.cache_image_int8(k, v, cu)
    np.testing.assert_array_equal(kq.cpu().numpy(), rk, err_msg=what + " k codes")
    np.testing.assert_array_equal(vq.cpu().numpy(), rv, err_msg=what + " v codes")
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32), err_msg=what + " k scales")
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32), err_msg=what + " v scales")


@pytest.mark.parametrize("H,HK,D", [(3, 3, 32), (4, 4, 64), (2, 2, 128), (8, 2, 128), (4, 1, 64)])
def test_int8_varlen_ragged(H, HK, D):
    lengths = [1, 70, 129, 0, 200, 64]
    g = I.generator(700 + H + HK + D)
    N = sum(lengths)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    cu = I.cu_from_lengths(lengths)
    scale = I.default_scale(D)
    say("case int8 varlen lengths=%s H=%d HK=%d D=%d" % (lengths, H, HK, D))
    out, kq, vq, ks, vs = run_int8(q, k, v, cu, scale)
    ref, _, _, _ = oracle.prefill_varlen(q, k, v, cu, scale)
    assert_close(out, ref, "int8 varlen out")
    check_codes(k, v, cu, kq, vq, ks, vs, "int8 varlen")


@pytest.mark.parametrize("D", [64, 128])
def test_int8_special_rows(D):
    """Zero rows, rows below 2^-100, wide dynamic range, exact ties (amax =
    127/64 so 127/amax = 64 and odd multiples of 1/128 land on .5)."""
    H = 2
    lengths = [40, 25]
    N = sum(lengths)
    g = I.generator(710)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, H, D))
    v = I.randn_bf16(g, (N, H, D))
    k[3, 0] = 0
    v[4, 1] = 0
    k[5, 1] = 1e-35
    gen = torch.Generator().manual_seed(711)
    # 36 decades: the smallest entries quantise to 0 (scores stay inside the
    # kernel's supported range |scale q.k| < 2^26)
    k[6, 0] = (torch.randn(D, generator=gen) * torch.logspace(-30, 6, D)).to(torch.bfloat16)
    ties = torch.tensor([127 / 64.0] + [(2 * i + 1) / 128.0 * (-1) ** i for i in range(D - 1)])
    k[7, 0] = ties.to(torch.bfloat16)
    v[8, 1] = (-ties).to(torch.bfloat16)
    cu = I.cu_from_lengths(lengths)
    say("case int8 special rows")
    out, kq, vq, ks, vs = run_int8(q, k, v, cu, 0.125)
    check_codes(k, v, cu, kq, vq, ks, vs, "int8 special")
    ref, _, _, _ = oracle.prefill_varlen(q, k, v, cu, 0.125)
    assert_close(out, ref, "int8 special out")


def test_int8_dequantised_cache_within_half_step():
    """Independent of the oracle: every cached value is within half a
    quantisation step of the bf16 value it encodes, and the largest |x| of
    each row encodes as +-127."""
    H, HK, D = 4, 2, 128
    lengths = [300, 17]
    N = sum(lengths)
    g = I.generator(720)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    cu = I.cu_from_lengths(lengths)
    _, kq, vq, ks, vs = run_int8(q, k, v, cu, 0.1)
    z = np.zeros(N * HK * D, np.uint16)
    kimg, _ = oracle.cache_image(k, v, cu, z, z)  # bf16 placement only
    x = torch.from_numpy(kimg.view(np.int16)).view(torch.bfloat16).float().double().numpy().reshape(-1, D)
    c = kq.cpu().numpy().astype(np.float64).reshape(-1, D)
    s = ks.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(x - c * s[:, None]) <= 0.5 * s[:, None] * (1 + 2.0 ** -20) + 2.0 ** -22 * np.abs(x))
    top = c[np.arange(c.shape[0]), np.abs(x).argmax(axis=1)]
    assert np.all(np.abs(top) == 127)


def test_int8_T2048_H32_D128():
    """The single-sequence workload (T=2048, 32 heads x 128): whole INT8 cache
    bit for bit, sampled output rows against the oracle."""
    w = I.workload("single_T2048_H32_D128")
    q, k, v = w.tensors()
    say("case int8 %s" % w.name)
    out, kq, vq, ks, vs = run_int8(q, k, v, w.cu_seqlens, w.scale)
    check_codes(k, v, w.cu_seqlens, kq, vq, ks, vs, "int8 T2048")
    rows = [0, 1, 63, 64, 127, 128, 1000, 1023, 1024, 2046, 2047]
    ref = oracle.prefill_rows(q, k, v, w.cu_seqlens, w.scale, rows)
    assert_close(out[rows], ref, "int8 T2048 sampled")
