"""GPU parity for split-KV chunked prefill over a paged KV cache
(prefill_attn_chunked_splitkv_paged): 16-token blocks located through a block
table ("大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.2; untitled page
www.zwxr.cn/news/300951 §3.4).  Outputs against oracle.prefill_chunked_paged to
the parity bar of tests/gpu_util.py, the whole block pool bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import SENTINEL, assert_close, bits, say

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


def make_case(lengths, prefix, max_blocks, H, HK, D, seed, spare=5):
    """Inputs, a pool with every block randomly placed (plus unused spare
    blocks holding the sentinel) and its block table."""
    g = I.generator(seed)
    cu = I.cu_from_lengths(lengths)
    N, B = cu[-1], len(lengths)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    nb = B * max_blocks + spare
    perm = np.random.default_rng(seed).permutation(nb)[:B * max_blocks]
    bt = perm.reshape(B, max_blocks).astype(np.int32)
    kp = I.randn_bf16(g, (nb, HK, 16, D))
    vp = I.randn_bf16(g, (nb, HK, 16, D))
    sent = torch.tensor(SENTINEL, dtype=torch.int16).view(torch.bfloat16)
    used = set(bt.reshape(-1).tolist())
    for n in range(nb):
        if n not in used:
            kp[n] = sent
            vp[n] = sent
    return q, k, v, cu, bt, kp, vp


def run_paged(q, k, v, cu, pre, bt, kp, vp, scale, max_seqlen=None):
    kpd, vpd = kp.cuda(), vp.cuda()
    out = torch.empty_like(q, device="cuda")
    P().prefill_attn_chunked_splitkv_paged(
        q.cuda(), k.cuda(), v.cuda(), torch.tensor(cu, dtype=torch.int32, device="cuda"), kpd, vpd,
        torch.from_numpy(bt).cuda(), out, torch.tensor(pre, dtype=torch.int32, device="cuda"),
        scale=scale, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return out, kpd, vpd


LENGTHS = [1, 100, 1, 257, 64, 0, 1, 1, 1, 130, 3]
PREFIX = [0, 2000, 2500, 960, 1024, 10, 1023, 1024, 2047, 894, 2900]


@pytest.mark.parametrize("D", [32, 64, 128])
def test_paged_permuted_blocks_full(D):
    q, k, v, cu, bt, kp, vp = make_case(LENGTHS, PREFIX, 190, 3, 3, D, 1000 + D)
    scale = I.default_scale(D)
    say("case paged D=%d blocks=%d" % (D, kp.shape[0]))
    out, kpd, vpd = run_paged(q, k, v, cu, PREFIX, bt, kp, vp, scale)
    ref, kimg, vimg = oracle.prefill_chunked_paged(q, k, v, cu, PREFIX, kp, vp, bt, scale)
    assert_close(out, ref, "paged D=%d" % D)
    np.testing.assert_array_equal(bits(kpd), kimg)
    np.testing.assert_array_equal(bits(vpd), vimg)


@pytest.mark.parametrize("H,HK,D", [(8, 2, 128), (16, 2, 64)])
def test_paged_grouped_heads(H, HK, D):
    lengths, prefix = [96, 1, 1, 33, 1], [1500, 3000, 1, 64, 2048]
    q, k, v, cu, bt, kp, vp = make_case(lengths, prefix, 200, H, HK, D, 1010 + H + D)
    say("case paged gqa H=%d HK=%d D=%d" % (H, HK, D))
    out, kpd, vpd = run_paged(q, k, v, cu, prefix, bt, kp, vp, 0.1)
    ref, kimg, vimg = oracle.prefill_chunked_paged(q, k, v, cu, prefix, kp, vp, bt, 0.1)
    assert_close(out, ref, "paged gqa")
    np.testing.assert_array_equal(bits(kpd), kimg)
    np.testing.assert_array_equal(bits(vpd), vimg)


def test_paged_shared_prefix_blocks():
    """Four requests share one 1040-token prefix (65 blocks); each has its own
    blocks for what follows (two chunks, two decode rows)."""
    H, D, pre = 4, 128, 1040
    g = I.generator(1020)
    lengths = [50, 1, 17, 1]
    cu = I.cu_from_lengths(lengths)
    N = cu[-1]
    q, k, v = (I.randn_bf16(g, (N, H, D)) for _ in range(3))
    shared = 65
    mb = 70
    nb = shared + 4 * (mb - shared)
    bt = np.zeros((4, mb), np.int32)
    for b in range(4):
        bt[b, :shared] = np.arange(shared)
        bt[b, shared:] = shared + b * (mb - shared) + np.arange(mb - shared)
    kp = I.randn_bf16(g, (nb, H, 16, D))
    vp = I.randn_bf16(g, (nb, H, 16, D))
    say("case paged shared prefix")
    out, kpd, vpd = run_paged(q, k, v, cu, [pre] * 4, bt, kp, vp, 0.09)
    ref, kimg, vimg = oracle.prefill_chunked_paged(q, k, v, cu, [pre] * 4, kp, vp, bt, 0.09)
    assert_close(out, ref, "paged shared prefix")
    np.testing.assert_array_equal(bits(kpd), kimg)
    np.testing.assert_array_equal(bits(vpd), vimg)


def test_paged_matches_slab_bitwise():
    """The same problem through the slab layout and through a permuted paged
    layout of equal capacity: identical output bits (same work split, same
    arithmetic), cache contents the same positions."""
    lengths, prefix, mb, H, D = [200, 1, 1, 17], [1800, 4000, 700, 3000], 257, 4, 128
    q, k, v, cu, bt, kp, vp = make_case(lengths, prefix, mb, H, H, D, 1030, spare=0)
    B, cap = len(lengths), 16 * mb
    slab_k = torch.empty((B, H, cap, D), dtype=torch.bfloat16)
    slab_v = torch.empty_like(slab_k)
    for b in range(B):
        for i in range(mb):
            slab_k[b, :, 16 * i:16 * (i + 1)] = kp[bt[b, i]]
            slab_v[b, :, 16 * i:16 * (i + 1)] = vp[bt[b, i]]
    out_p, kpd, _ = run_paged(q, k, v, cu, prefix, bt, kp, vp, 0.08)
    kc, vc = slab_k.cuda(), slab_v.cuda()
    out_s = torch.empty_like(q, device="cuda")
    P().prefill_attn_chunked_splitkv(q.cuda(), k.cuda(), v.cuda(),
                                     torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc,
                                     out_s, torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                                     scale=0.08)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out_p), bits(out_s))
    kb = bits(kpd)
    sb = bits(kc)
    for b in range(B):
        for i in range(mb):
            np.testing.assert_array_equal(kb[bt[b, i]], sb[b, :, 16 * i:16 * (i + 1)])


def test_paged_check_mode_rejects_block_outside_pool():
    lib = P().load()
    H, D = 2, 64
    q = torch.zeros((4, H, D), dtype=torch.bfloat16, device="cuda")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    out = torch.ones_like(q)
    kp = torch.zeros((3, H, 16, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    pre = torch.tensor([20], dtype=torch.int32, device="cuda")
    bt_bad = torch.tensor([[0, 3]], dtype=torch.int32, device="cuda")  # block 3 of a pool of 3
    ws = torch.zeros(P().splitkv_workspace_size(1, 4, H, D, 32), dtype=torch.uint8, device="cuda")
    prev = P().pa_set_check_mode(True)
    try:
        st = lib.prefill_attn_chunked_splitkv_paged(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(), 1, 4, 4, H, H, D,
            kp.data_ptr(), vp.data_ptr(), 3, bt_bad.data_ptr(), 2, out.data_ptr(),
            ctypes.c_float(0.1), torch.cuda.current_stream().cuda_stream, pre.data_ptr(),
            ws.data_ptr(), ws.numel())
        assert st == 8
        torch.cuda.synchronize()
        assert bool(torch.all(out == 1)), "a rejected call wrote its output"
    finally:
        P().pa_set_check_mode(prev)
