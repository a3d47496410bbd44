"""Randomised GPU parity sweep: small batches with random lengths, prefixes,
head groupings, head sizes and scales through every entry point of the C ABI
(varlen, INT8- and FP8-cache varlen, one-pass chunked, split-KV chunked over a slab
and over a paged pool), each against the float64 oracle: outputs to the
parity bar of tests/gpu_util.py, caches bit for bit.  Seeded, so a failure
names its case and reproduces."""
import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import SENTINEL, assert_close, bits, say

pytestmark = pytest.mark.gpu

CASES = 24


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


def draw_case(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([32, 64, 128]))
    HK = int(rng.choice([1, 2, 3]))
    H = HK * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 7))
    lengths, prefix = [], []
    for _ in range(B):
        kind = rng.random()
        if kind < 0.35:
            lengths.append(1)                                   # decode row
        elif kind < 0.45:
            lengths.append(0)                                   # empty
        else:
            lengths.append(int(rng.integers(2, 300)))           # chunk
        prefix.append(int(rng.integers(0, 2600)) if rng.random() < 0.8 else 0)
    scale = float(rng.choice([I.default_scale(D), 0.0, -0.2, 0.7]))
    return dict(D=D, H=H, HK=HK, lengths=lengths, prefix=prefix, scale=scale)


def tensors(c, seed):
    g = I.generator(seed)
    cu = I.cu_from_lengths(c["lengths"])
    N = cu[-1]
    q = I.randn_bf16(g, (N, c["H"], c["D"]))
    k = I.randn_bf16(g, (N, c["HK"], c["D"]))
    v = I.randn_bf16(g, (N, c["HK"], c["D"]))
    return q, k, v, cu


@pytest.mark.parametrize("i", range(CASES))
def test_random_chunked_paths(i):
    seed = 5000 + i
    c = draw_case(seed)
    q, k, v, cu = tensors(c, seed)
    B, D, HK = len(c["lengths"]), c["D"], c["HK"]
    cap = 16 * ((max(p + n for p, n in zip(c["prefix"], c["lengths"])) + 15) // 16 + 1)
    g = I.generator(seed + 1)
    kc0 = I.randn_bf16(g, (B, HK, cap, D))
    vc0 = I.randn_bf16(g, (B, HK, cap, D))
    say("case %d: %s cap=%d" % (i, c, cap))
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, c["prefix"], kc0, vc0, c["scale"])
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    pred = torch.tensor(c["prefix"], dtype=torch.int32, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()

    # one-pass chunked
    kc, vc = kc0.cuda(), vc0.cuda()
    out = torch.empty_like(qd)
    P().prefill_attn_chunked(qd, kd, vd, cud, kc, vc, out, pred, scale=c["scale"])
    torch.cuda.synchronize()
    assert_close(out, ref, "case %d one-pass" % i)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)

    # split-KV over the slab
    kc, vc = kc0.cuda(), vc0.cuda()
    out = torch.empty_like(qd)
    P().prefill_attn_chunked_splitkv(qd, kd, vd, cud, kc, vc, out, pred, scale=c["scale"])
    torch.cuda.synchronize()
    assert_close(out, ref, "case %d split-KV" % i)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)

    # split-KV over a paged pool (blocks shuffled, two spare blocks of sentinel)
    mb = cap // 16
    perm = np.random.default_rng(seed + 2).permutation(B * mb + 2)
    bt = perm[:B * mb].reshape(B, mb).astype(np.int32)
    sent = torch.tensor(SENTINEL, dtype=torch.int16).view(torch.bfloat16)
    kp = torch.full((B * mb + 2, HK, 16, D), float("nan"), dtype=torch.bfloat16)
    kp[:] = sent
    vp = kp.clone()
    for b in range(B):
        for j in range(mb):
            kp[bt[b, j]] = kc0[b, :, 16 * j:16 * (j + 1)]
            vp[bt[b, j]] = vc0[b, :, 16 * j:16 * (j + 1)]
    kpd, vpd = kp.cuda(), vp.cuda()
    out = torch.empty_like(qd)
    P().prefill_attn_chunked_splitkv_paged(qd, kd, vd, cud, kpd, vpd, torch.from_numpy(bt).cuda(), out, pred,
                                           scale=c["scale"])
    torch.cuda.synchronize()
    pref, pk_img, pv_img = oracle.prefill_chunked_paged(q, k, v, cu, c["prefix"], kp, vp, bt, c["scale"])
    assert_close(out, pref, "case %d paged" % i)
    np.testing.assert_array_equal(bits(kpd), pk_img)
    np.testing.assert_array_equal(bits(vpd), pv_img)


@pytest.mark.parametrize("i", range(CASES))
def test_random_varlen_paths(i):
    seed = 6000 + i
    c = draw_case(seed)
    lengths = [n if n > 1 else n + int(np.random.default_rng(seed).integers(0, 200)) for n in c["lengths"]]
    q, k, v, cu = tensors(dict(c, lengths=lengths), seed)
    N, H, D = q.shape
    HK = k.shape[1]
    say("case %d: lengths=%s H=%d HK=%d D=%d scale=%g" % (i, lengths, H, HK, D, c["scale"]))
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sent = np.full(N * HK * D, SENTINEL, np.uint16)
    ref, kimg, vimg, _ = oracle.prefill_varlen(q, k, v, cu, c["scale"], k_cache=sent, v_cache=sent)

    kc = torch.full((N * HK * D,), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vc = kc.clone()
    out = torch.empty_like(qd)
    P().prefill_attn_varlen(qd, kd, vd, cud, kc, vc, out, scale=c["scale"])
    torch.cuda.synchronize()
    assert_close(out, ref, "case %d varlen" % i)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)

    kq = torch.zeros(N * HK * D, dtype=torch.int8, device="cuda")
    vq = torch.zeros_like(kq)
    ks = torch.zeros(N * HK, dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    out = torch.empty_like(qd)
    P().prefill_attn_varlen_int8(qd, kd, vd, cud, kq, vq, ks, vs, out, scale=c["scale"])
    torch.cuda.synchronize()
    assert_close(out, ref, "case %d varlen INT8" % i)
    rk, rks, rv, rvs = oracle.cache_image_int8(k, v, cu)
    np.testing.assert_array_equal(kq.cpu().numpy(), rk)
    np.testing.assert_array_equal(vq.cpu().numpy(), rv)
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32))

    kf, vf = kq.view(torch.uint8), vq.view(torch.uint8)
    out = torch.empty_like(qd)
    P().prefill_attn_varlen_fp8(qd, kd, vd, cud, kf, vf, ks, vs, out, scale=c["scale"])
    torch.cuda.synchronize()
    assert_close(out, ref, "case %d varlen FP8" % i)
    rk, rks, rv, rvs = oracle.cache_image_fp8(k, v, cu)
    np.testing.assert_array_equal(kf.cpu().numpy(), rk)
    np.testing.assert_array_equal(vf.cpu().numpy(), rv)
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32))
