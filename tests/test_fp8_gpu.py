"""GPU parity for the FP8 KV-cache write (prefill_attn_varlen_fp8): attention
outputs against the float64 oracle to the parity bar of tests/gpu_util.py,
E4M3 codes and float scales bit for bit against oracle.cache_image_fp8
("大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.3: K and V quantised,
Q kept; the oracle fixes the E4M3 reading and the per-row scale), guard bands
around every output untouched."""
import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import assert_close, say

pytestmark = pytest.mark.gpu

GUARD = 4096
BYTE_SENTINEL = 0x5A  # an E4M3 code (72.0), never NaN
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


def guarded_u8(n):
    whole = torch.full((n + 2 * GUARD,), BYTE_SENTINEL, dtype=torch.uint8, device="cuda")
    return whole[GUARD:GUARD + n], whole


def guarded_f32(n):
    whole = torch.full((n + 2 * GUARD,), F32_SENTINEL, dtype=torch.int32, device="cuda")
    return whole[GUARD:GUARD + n].view(torch.float32), whole


def guards_ok(whole, sentinel):
    a = whole.cpu().numpy()
    return bool(np.all(a[:GUARD] == sentinel) and np.all(a[-GUARD:] == sentinel))


def run_fp8(q, k, v, cu, scale):
    N, H, D = q.shape
    HK = k.shape[1]
    kq, kq_w = guarded_u8(N * HK * D)
    vq, vq_w = guarded_u8(N * HK * D)
    ks, ks_w = guarded_f32(N * HK)
    vs, vs_w = guarded_f32(N * HK)
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    P().prefill_attn_varlen_fp8(q.cuda(), k.cuda(), v.cuda(),
                                 torch.tensor(cu, dtype=torch.int32, device="cuda"),
                                 kq, vq, ks, vs, out, scale=scale)
    torch.cuda.synchronize()
    assert guards_ok(kq_w, BYTE_SENTINEL) and guards_ok(vq_w, BYTE_SENTINEL)
    assert guards_ok(ks_w, F32_SENTINEL) and guards_ok(vs_w, F32_SENTINEL)
    return out, kq, vq, ks, vs


def check_codes(k, v, cu, kq, vq, ks, vs, what):
    rk, rks, rv, rvs = oracle.cache_image_fp8(k, v, cu)
    np.testing.assert_array_equal(kq.cpu().numpy(), rk, err_msg=what + " k codes")
    np.testing.assert_array_equal(vq.cpu().numpy(), rv, err_msg=what + " v codes")
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32), err_msg=what + " k scales")
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32), err_msg=what + " v scales")


@pytest.mark.parametrize("H,HK,D", [(3, 3, 32), (4, 4, 64), (2, 2, 128), (8, 2, 128), (4, 1, 64)])
def test_fp8_varlen_ragged(H, HK, D):
    lengths = [1, 70, 129, 0, 200, 64]
    g = I.generator(700 + H + HK + D)
    N = sum(lengths)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    cu = I.cu_from_lengths(lengths)
    scale = I.default_scale(D)
    say("case fp8 varlen lengths=%s H=%d HK=%d D=%d" % (lengths, H, HK, D))
    out, kq, vq, ks, vs = run_fp8(q, k, v, cu, scale)
    ref, _, _, _ = oracle.prefill_varlen(q, k, v, cu, scale)
    assert_close(out, ref, "fp8 varlen out")
    check_codes(k, v, cu, kq, vq, ks, vs, "fp8 varlen")


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_special_rows(D):
    """Zero rows (codes keep the sign of x * 0), rows below 2^-100, a wide
    dynamic range reaching the E4M3 subnormals, exact midpoints (amax = 448
    gives scale 1, and values halfway between neighbouring E4M3 codes)."""
    H = 2
    lengths = [40, 25]
    N = sum(lengths)
    g = I.generator(810)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, H, D))
    v = I.randn_bf16(g, (N, H, D))
    k[3, 0] = 0
    v[4, 1] = -0.0
    k[5, 1] = 1e-35
    gen = torch.Generator().manual_seed(811)
    k[6, 0] = (torch.randn(D, generator=gen) * torch.logspace(-30, 6, D)).to(torch.bfloat16)
    # midpoints between neighbouring codes, all exact in bf16 (at most 5
    # significant bits); 448 first so the scale is exactly 1; codes 0x28 ..
    # 0x7d, again from 0x28 when D - 1 passes them (0x7e is 448, 0x7f NaN)
    mids = [448.0] + [(oracle.e4m3_decode(c) + oracle.e4m3_decode(c + 1)) / 2 * (-1) ** c
                      for c in (0x28 + i % 0x55 for i in range(D - 1))]
    ties = torch.tensor(mids)
    k[7, 0] = ties.to(torch.bfloat16)
    v[8, 1] = (-ties).to(torch.bfloat16)
    assert torch.equal(k[7, 0].float(), ties.float())
    cu = I.cu_from_lengths(lengths)
    say("case fp8 special rows")
    out, kq, vq, ks, vs = run_fp8(q, k, v, cu, 0.125)
    check_codes(k, v, cu, kq, vq, ks, vs, "fp8 special")
    ref, _, _, _ = oracle.prefill_varlen(q, k, v, cu, 0.125)
    assert_close(out, ref, "fp8 special out")


def test_fp8_dequantised_cache_within_half_step():
    """Independent of the oracle's encoder: every cached value, decoded from
    the E4M3 definition and scaled, is within half a step of the bf16 value
    it encodes (2^-4 relative for normals, 2^-10 of the scale below 2^-6),
    and the largest |x| of each row encodes as +-448."""
    H, HK, D = 4, 2, 128
    lengths = [300, 17]
    N = sum(lengths)
    g = I.generator(820)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    cu = I.cu_from_lengths(lengths)
    _, kq, vq, ks, vs = run_fp8(q, k, v, cu, 0.1)
    z = np.zeros(N * HK * D, np.uint16)
    kimg, _ = oracle.cache_image(k, v, cu, z, z)  # bf16 placement only
    x = torch.from_numpy(kimg.view(np.int16)).view(torch.bfloat16).float().double().numpy().reshape(-1, D)
    codes = kq.cpu().numpy().reshape(-1, D)
    sgn = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 15
    m = (codes & 7).astype(np.float64)
    val = sgn * np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * 2.0 ** (e.astype(np.float64) - 7))
    s = ks.cpu().numpy().astype(np.float64)
    y = x / s[:, None]
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 2.0 ** -20) + np.abs(y) * 2.0 ** -22
    assert np.all(np.abs(val - y) <= bound)
    top = codes[np.arange(codes.shape[0]), np.abs(x).argmax(axis=1)]
    assert np.all((top & 0x7F) == 0x7E)


def test_fp8_T2048_H32_D128():
    """The single-sequence workload (T=2048, 32 heads x 128): whole FP8 cache
    bit for bit, sampled output rows against the oracle."""
    w = I.workload("single_T2048_H32_D128")
    q, k, v = w.tensors()
    say("case fp8 %s" % w.name)
    out, kq, vq, ks, vs = run_fp8(q, k, v, w.cu_seqlens, w.scale)
    check_codes(k, v, w.cu_seqlens, kq, vq, ks, vs, "fp8 T2048")
    rows = [0, 1, 63, 64, 127, 128, 1000, 1023, 1024, 2046, 2047]
    ref = oracle.prefill_rows(q, k, v, w.cu_seqlens, w.scale, rows)
    assert_close(out[rows], ref, "fp8 T2048 sampled")
