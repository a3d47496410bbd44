"""GPU parity for split-KV chunked prefill (prefill_attn_chunked_splitkv): the
keys of each query block are cut into segments of >= 1024 keys, each an
independent work item, and blocks with several segments are finished by a
log-sum-exp merge.  The result is the chunked attention of the pages
("大模型 Prompt Prefill 阶段的高效 Batching 与算子排布" §3: a prompt chunk batched
with decode rows; untitled page www.zwxr.cn/news/300951 §3.3: a decode row
reads its whole cache), so the oracle is oracle.prefill_chunked: outputs to
the parity bar of tests/gpu_util.py, cache bytes bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import SENTINEL, assert_close, bits, guards_intact, say

pytestmark = pytest.mark.gpu

WS_GUARD = 4096  # bytes after the workspace that must stay untouched


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


def sentinel_cache(g, B, HK, cap, D, prefix):
    """Random cache with the sentinel at and beyond each prefix (stray writes show)."""
    c = I.randn_bf16(g, (B, HK, cap, D))
    s = torch.tensor(SENTINEL, dtype=torch.int16).view(torch.bfloat16)
    for b, p in enumerate(prefix):
        c[b, :, p:] = s
    return c


def workspace_for(B, N, H, D, cap, fill=0xFF):
    need = P().splitkv_workspace_size(B, N, H, D, cap)
    assert need > 0
    whole = torch.full((need + WS_GUARD,), fill, dtype=torch.uint8, device="cuda")
    return whole, need


def run_split(q, k, v, cu, pre, kc, vc, scale, ws=None, max_seqlen=None):
    out = torch.empty_like(q, device="cuda")
    P().prefill_attn_chunked_splitkv(
        q.cuda(), k.cuda(), v.cuda(), torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc,
        out, torch.tensor(pre, dtype=torch.int32, device="cuda"), scale=scale,
        max_seqlen=max_seqlen, workspace=ws)
    torch.cuda.synchronize()
    return out


def check_case(lengths, prefix, cap, H, HK, D, seed, what, scale=None, max_seqlen=None):
    g = I.generator(seed)
    cu = I.cu_from_lengths(lengths)
    N, B = cu[-1], len(lengths)
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, HK, D))
    v = I.randn_bf16(g, (N, HK, D))
    kc0 = sentinel_cache(g, B, HK, cap, D, prefix)
    vc0 = sentinel_cache(g, B, HK, cap, D, prefix)
    scale = I.default_scale(D) if scale is None else scale
    say("case %s: lengths=%s prefix=%s cap=%d H=%d HK=%d D=%d scale=%g"
        % (what, lengths, prefix, cap, H, HK, D, scale))
    whole, need = workspace_for(B, N, H, D, cap)
    kc, vc = kc0.cuda(), vc0.cuda()
    out = run_split(q, k, v, cu, prefix, kc, vc, scale, ws=whole[:need], max_seqlen=max_seqlen)
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, prefix, kc0, vc0, scale)
    assert_close(out, ref, what)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)
    assert bool(torch.all(whole[need:] == 0xFF)), "write past the workspace"
    return q, k, v, cu, kc0, vc0, out


# prefixes around the 1024-key segment edges: a block whose last segment holds
# no key of its first rows (960 + 128 rows), keys ending exactly on a segment
# edge (1023 + 1, 2047 + 1), a decode row with no prefix
LENGTHS = [1, 100, 1, 257, 64, 0, 1, 1, 1, 130, 3]
PREFIX = [0, 2000, 2500, 960, 1024, 10, 1023, 1024, 2047, 894, 2900]


@pytest.mark.parametrize("D", [32, 64, 128])
def test_splitkv_segment_edges_full(D):
    check_case(LENGTHS, PREFIX, 3000, 3, 3, D, 900 + D, "splitkv edges D=%d" % D)


@pytest.mark.parametrize("H,HK,D", [(8, 2, 128), (4, 1, 64), (16, 2, 64), (6, 3, 32), (32, 1, 128), (8, 4, 128)])
def test_splitkv_grouped_heads(H, HK, D):
    # decode rows share each K/V load among 4, 4, 8, 2, 8 and 2 query heads
    # (1 or 2: the rows run inside the attention launch, else in their own)
    check_case([96, 1, 1, 33, 1], [1500, 3000, 1, 64, 2048], 3100, H, HK, D, 910 + H + D,
               "splitkv gqa H=%d HK=%d" % (H, HK))


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
def test_splitkv_other_scales(scale):
    check_case([1, 70, 1], [1500, 1100, 3], 1600, 4, 4, 64, 950, "splitkv scale", scale=scale)


def test_splitkv_decode_rows_only():
    """A batch of decode rows only (no prompt chunk), contexts across segment edges."""
    ctx = [0, 1, 63, 64, 1023, 1024, 1025, 2047, 2048, 4095, 5000]
    check_case([1] * len(ctx), ctx, 5001, 4, 4, 128, 960, "splitkv decode only")


def test_splitkv_decode_rows_only_larger_max_seqlen():
    """Only length-1 rows, but max_seqlen 4 (an upper bound, as the header
    allows): the launch that runs decode rows beside attention items gets no
    item, and every work-group starts on the decode units."""
    ctx = [0, 1, 64, 1023, 1024, 2047, 4095, 5000, 333]
    check_case([1] * len(ctx), ctx, 5001, 4, 4, 128, 965, "splitkv decode only, max_seqlen 4", max_seqlen=4)


def test_splitkv_batch_without_decode_rows():
    """Several multi-token sequences and no length-1 row: in the launch that
    runs decode rows beside attention items every work-group starts on the
    items (segments of 64 tiles: blocks with one, two and three segments)."""
    check_case([100, 40, 260, 2], [1500, 0, 8000, 77], 8300, 4, 4, 128, 985, "splitkv no decode rows")


def test_splitkv_long_context_many_segments():
    """Capacity 70000: more than 64 * 1024 keys, so segments grow to 18 tiles."""
    check_case([1, 1, 40], [69999, 35000, 66000], 70040, 2, 2, 64, 920, "splitkv 70k context")


def test_splitkv_matches_unsplit_chunked():
    """Same inputs through the one-pass chunked call: identical cache bytes,
    outputs within the parity bar of each other's oracle (both are checked)."""
    lengths, prefix, cap, H, D = [200, 1, 1, 17], [1800, 4000, 700, 3000], 4100, 4, 128
    q, k, v, cu, kc0, vc0, out_s = check_case(lengths, prefix, cap, H, H, D, 930, "splitkv vs chunked")
    kc, vc = kc0.cuda(), vc0.cuda()
    out_c = torch.empty_like(q, device="cuda")
    P().prefill_attn_chunked(q.cuda(), k.cuda(), v.cuda(),
                             torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc, out_c,
                             torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                             scale=I.default_scale(D))
    torch.cuda.synchronize()
    d = (out_s.float() - out_c.float()).abs().max().item()
    say("  splitkv vs chunked max |d| = %.3e" % d)
    assert d <= 2e-2


def test_splitkv_workspace_reused_smaller_second_call():
    """A workspace keeps nothing between calls: a large call then a smaller one
    on the same (garbage-filled) buffer both match the oracle."""
    cases = [([300, 1, 1], [3000, 5000, 100], 5400, 4, 64),
             ([1, 50], [2000, 1100], 2200, 4, 64)]
    big = max(P().splitkv_workspace_size(len(L), sum(L), H, D, cap) for L, _, cap, H, D in cases)
    ws = torch.full((big,), 0x7F, dtype=torch.uint8, device="cuda")
    for i, (lengths, prefix, cap, H, D) in enumerate(cases):
        g = I.generator(940 + i)
        cu = I.cu_from_lengths(lengths)
        N, B = cu[-1], len(lengths)
        q, k, v = (I.randn_bf16(g, (N, H, D)) for _ in range(3))
        kc0 = sentinel_cache(g, B, H, cap, D, prefix)
        vc0 = sentinel_cache(g, B, H, cap, D, prefix)
        say("case reuse call %d" % i)
        kc, vc = kc0.cuda(), vc0.cuda()
        out = run_split(q, k, v, cu, prefix, kc, vc, 0.1, ws=ws)
        ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, prefix, kc0, vc0, 0.1)
        assert_close(out, ref, "reuse call %d" % i)
        np.testing.assert_array_equal(bits(kc), kimg)


def test_splitkv_chunked_workload_steps():
    """8192-token prompt in 512-token chunks beside 64 decode rows: steps 0, 7
    and 15 (prefix 0, 3584, 7680) through the split path, sampled chunk rows
    and every decode row against the oracle, whole caches bit for bit."""
    wl = I.workload("chunked_8192x512_plus_64_decode_H32_D128")
    H, D, R = wl.num_heads, wl.head_dim, len(wl.contexts)
    say("case chunked workload via splitkv: drawing inputs")
    t = wl.tensors()
    B = 1 + R
    kc = torch.zeros((B, H, wl.cap, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for r, ctx in enumerate(wl.contexts):
        kc[1 + r, :, :ctx] = t["pre_k"][r].cuda()
        vc[1 + r, :, :ctx] = t["pre_v"][r].cuda()
    rng = np.random.default_rng(1)
    for c in range(wl.num_chunks):
        st = wl.step(c)
        sl = slice(c * wl.chunk_len, (c + 1) * wl.chunk_len)
        q = torch.cat([t["pq"][sl], t["dq"]])
        k = torch.cat([t["pk"][sl], t["dk"]])
        v = torch.cat([t["pv"][sl], t["dv"]])
        check = c in (0, 7, 15)
        kc_before = kc.cpu() if check else None
        vc_before = vc.cpu() if check else None
        say("  step %d" % c)
        out = run_split(q, k, v, st.cu_seqlens, st.prefix_lens, kc, vc, st.scale,
                        max_seqlen=wl.chunk_len)
        if not check:
            continue
        rows = sorted(set([0, 1, 63, 64, 127, 128, 255, 256, 511] +
                          rng.integers(0, 512, 24).tolist() + list(range(512, 512 + R))))
        ref = oracle.prefill_rows(q, k, v, st.cu_seqlens, st.scale, rows,
                                  prefix_lens=st.prefix_lens, k_cache=kc_before, v_cache=vc_before)
        assert_close(out[rows], ref, "splitkv chunk step %d" % c)
        kimg, vimg = oracle.cache_image(k, v, st.cu_seqlens, kc_before, vc_before,
                                        prefix_lens=st.prefix_lens)
        np.testing.assert_array_equal(bits(kc), kimg)
        np.testing.assert_array_equal(bits(vc), vimg)
    np.testing.assert_array_equal(bits(kc[0]), bits(t["pk"]).transpose(1, 0, 2))


def test_splitkv_check_mode_rejects_tokens_beyond_num_tokens():
    """Check mode: cu_seqlens[B] above num_tokens is PA_ERR_SEQLENS, nothing launched."""
    lib = P().load()
    H, D, cap = 2, 64, 64
    q = torch.zeros((8, H, D), dtype=torch.bfloat16, device="cuda")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    out = torch.ones_like(q)
    kc = torch.zeros((1, H, cap, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    cu = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    pre = torch.tensor([0], dtype=torch.int32, device="cuda")
    ws = torch.zeros(P().splitkv_workspace_size(1, 8, H, D, cap), dtype=torch.uint8, device="cuda")
    prev = P().pa_set_check_mode(True)
    try:
        st = lib.prefill_attn_chunked_splitkv(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(), 1, 8, 4, H, H, D,
            kc.data_ptr(), vc.data_ptr(), cap, out.data_ptr(), ctypes.c_float(0.1),
            torch.cuda.current_stream().cuda_stream, pre.data_ptr(), ws.data_ptr(), ws.numel())
        assert st == 7
        torch.cuda.synchronize()
        assert bool(torch.all(out == 1)), "a rejected call wrote its output"
        st = lib.prefill_attn_chunked_splitkv(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(), 1, 8, 8, H, H, D,
            kc.data_ptr(), vc.data_ptr(), cap, out.data_ptr(), ctypes.c_float(0.1),
            torch.cuda.current_stream().cuda_stream, pre.data_ptr(), ws.data_ptr(), ws.numel())
        assert st == 0
        torch.cuda.synchronize()
    finally:
        P().pa_set_check_mode(prev)
    assert bool(torch.all(out == 0)), "v = 0 gives out = 0"


def test_splitkv_thousands_of_rows():
    """2,100 sequences (the plan takes 1,024 per round): decode rows with
    contexts 0..1,090 (one or two segments), empty sequences and one chunk."""
    rng = np.random.default_rng(970)
    B = 2100
    lengths = [1] * B
    prefix = rng.integers(0, 1091, B).tolist()
    for b in (5, 1500, 2099):
        lengths[b] = 0
    lengths[1024] = 60          # a chunk in the second round
    prefix[1024] = 1000
    check_case(lengths, prefix, 1100, 2, 1, 32, 971, "splitkv 2100 rows")
