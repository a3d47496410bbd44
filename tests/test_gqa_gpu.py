"""GPU parity for grouped K/V heads (grouped-query / multi-query attention,
untitled page www.zwxr.cn/news/300951 §2.4): the HIP path through the C ABI
against the float64 oracle, outputs to the parity bar of tests/gpu_util.py,
cache bytes and guard bands bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import assert_close, bits, guarded, guards_intact, say, SENTINEL

pytestmark = pytest.mark.gpu


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


def draw(lengths, H, HK, D, seed):
    g = I.generator(seed)
    n = sum(lengths)
    return I.randn_bf16(g, (n, H, D)), I.randn_bf16(g, (n, HK, D)), I.randn_bf16(g, (n, HK, D))


@pytest.mark.parametrize("H,HK,D", [(8, 2, 128), (4, 1, 64), (6, 3, 32), (32, 8, 128)])
def test_gqa_varlen_ragged_full(H, HK, D):
    lengths = [1, 70, 129, 0, 200] if H < 32 else [10, 50, 300]
    q, k, v = draw(lengths, H, HK, D, 500 + H + HK + D)
    cu = I.cu_from_lengths(lengths)
    N = sum(lengths)
    scale = I.default_scale(D)
    say("case gqa varlen lengths=%s H=%d HK=%d D=%d" % (lengths, H, HK, D))
    out, out_w = guarded(N * H * D)
    kc, kc_w = guarded(N * HK * D)
    vc, vc_w = guarded(N * HK * D)
    P().prefill_attn_varlen(q.cuda(), k.cuda(), v.cuda(),
                            torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc,
                            out.view(N, H, D), scale=scale)
    torch.cuda.synchronize()
    sent = np.full(N * HK * D, SENTINEL, np.uint16)
    ref, kimg, vimg, _ = oracle.prefill_varlen(q, k, v, cu, scale, k_cache=sent, v_cache=sent)
    assert_close(out.view(N, H, D), ref, "gqa varlen")
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)
    assert all(guards_intact(w) for w in (out_w, kc_w, vc_w))


@pytest.mark.parametrize("H,HK,D", [(8, 2, 128), (4, 1, 64)])
def test_gqa_chunked_with_decode_rows(H, HK, D):
    """A prompt chunk and decode rows over cached prefixes, grouped K/V heads."""
    lengths = [96, 1, 1, 33]
    prefixes = [130, 300, 1, 64]
    cap = 512
    q, k, v = draw(lengths, H, HK, D, 600 + H + HK + D)
    g = I.generator(601 + D)
    B = len(lengths)
    kc0 = I.randn_bf16(g, (B, HK, cap, D))
    vc0 = I.randn_bf16(g, (B, HK, cap, D))
    cu = I.cu_from_lengths(lengths)
    scale = I.default_scale(D)
    say("case gqa chunked H=%d HK=%d D=%d" % (H, HK, D))
    kc, vc = kc0.cuda(), vc0.cuda()
    out = torch.empty_like(q, device="cuda")
    P().prefill_attn_chunked(q.cuda(), k.cuda(), v.cuda(),
                             torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc, out,
                             torch.tensor(prefixes, dtype=torch.int32, device="cuda"),
                             scale=scale)
    torch.cuda.synchronize()
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, prefixes, kc0, vc0, scale)
    assert_close(out, ref, "gqa chunked")
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)


def test_gqa_T2048_H32_HK8_D128_sampled():
    """The single-sequence size with 8 K/V heads, in the bench's launch
    configuration: sampled rows (every head) and the whole cache image."""
    T, H, HK, D = 2048, 32, 8, 128
    q, k, v = draw([T], H, HK, D, 700)
    cu = [0, T]
    scale = I.default_scale(D)
    say("case gqa T2048 H32 HK8")
    kc = torch.empty((T * HK * D,), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    P().prefill_attn_varlen(q.cuda(), k.cuda(), v.cuda(),
                            torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc, out,
                            scale=scale, max_seqlen=T)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 127, 128, 1000, 1023, 1024, 2046, 2047]
    ref = oracle.prefill_rows(q, k, v, cu, scale, rows)
    assert_close(out[rows], ref, "gqa T2048 rows")
    sent = np.zeros(T * HK * D, np.uint16)
    kimg, vimg = oracle.cache_image(k, v, cu, sent, sent)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)


def test_gqa_rejects_heads_that_do_not_divide():
    q, k, v = draw([16], 6, 4, 64, 800)
    kc = torch.empty((16 * 4 * 64,), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.empty((16, 6, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P().PrefillAttnError):
        P().prefill_attn_varlen(q.cuda(), k.cuda(), v.cuda(),
                                torch.tensor([0, 16], dtype=torch.int32, device="cuda"), kc, vc,
                                out, max_seqlen=16)
