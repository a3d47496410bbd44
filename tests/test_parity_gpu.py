"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Outputs within |gpu - oracle| <= 1e-2 + 2e-2 |oracle| (tests/gpu_util.py);
KV-cache bytes, guard bands and exact-copy rows bit for bit.  Small problems
are compared element by element; the full-size workloads in the launch
configuration the bench times are compared in full where the oracle finishes
in seconds, else on sampled rows (every head), with the whole cache image
checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import (assert_close, bits, guarded, guards_intact, say, to_f64,
                            SENTINEL)

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


def run_varlen(q, k, v, cu, scale, max_seqlen=None):
    """Run the HIP varlen path; returns (out, kc, vc, wholes) on the device."""
    N, H, D = q.shape
    n = N * H * D
    out, out_w = guarded(n)
    kc, kc_w = guarded(n)
    vc, vc_w = guarded(n)
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    P().prefill_attn_varlen(q.cuda(), k.cuda(), v.cuda(), cu_d, kc, vc, out.view(N, H, D),
                            scale=scale, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return out.view(N, H, D), kc, vc, (out_w, kc_w, vc_w)


def check_varlen(lengths, H, D, seed, scale=None, q=None, k=None, v=None, what=""):
    w = I.Varlen("t", lengths, H, D, seed=seed)
    if q is None:
        q, k, v = w.tensors()
    scale = w.scale if scale is None else scale
    say("case %s lengths=%s H=%d D=%d seed=%d" % (what, lengths[:8], H, D, seed))
    out, kc, vc, wholes = run_varlen(q, k, v, w.cu_seqlens, scale)
    n = w.num_tokens * H * D
    sent = np.full(n, SENTINEL, np.uint16)
    ref, kimg, vimg, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, scale,
                                               k_cache=sent, v_cache=sent)
    assert_close(out, ref, what)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)
    assert all(guards_intact(x) for x in wholes)
    # first row of every non-empty sequence is an exact copy of its V row
    vb = bits(v)
    ob = bits(out)
    for b, L in enumerate(lengths):
        if L:
            s = w.cu_seqlens[b]
            np.testing.assert_array_equal(ob[s], vb[s])
    return w, q, k, v, out


# ---------------------------------------------------------------- small, full oracle

@pytest.mark.parametrize("D", [32, 64, 128])
def test_varlen_ragged_full(D):
    check_varlen([1, 37, 64, 65, 128, 129, 300, 0, 511, 2], 3, D, 100 + D, what="ragged D=%d" % D)


def test_single_T64_H4_D32():
    w = I.workload("single_T64_H4_D32")
    check_varlen(w.lengths, w.num_heads, w.head_dim, w.seed, what=w.name)


def test_varlen_10_50_2048_H32_D128():
    w = I.workload("varlen_10_50_2048_H32_D128")
    check_varlen(w.lengths, w.num_heads, w.head_dim, w.seed, what=w.name)


def test_single_T2048_H32_D128():
    w = I.workload("single_T2048_H32_D128")
    check_varlen(w.lengths, w.num_heads, w.head_dim, w.seed, what=w.name)


def test_length_one_sequences_return_v_exactly():
    w = I.Varlen("t", [1] * 40, 8, 128, seed=7)
    q, k, v = w.tensors()
    out, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    np.testing.assert_array_equal(bits(out), bits(v))


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_other_scales(scale):
    check_varlen([5, 130, 257], 2, 64, 8, scale=scale, what="scale=%g" % scale)


def test_identical_keys_running_mean():
    w = I.Varlen("t", [200, 33], 2, 128, seed=9)
    q, k, v = w.tensors()
    k = k.clone()
    k[:200] = k[0]
    k[200:] = k[200]
    out, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    V = to_f64(v)
    for s, e in ((0, 200), (200, 233)):
        mean = np.cumsum(V[s:e], axis=0) / np.arange(1, e - s + 1)[:, None, None]
        assert_close(out[s:e], mean, "running mean")


def test_v_ones_gives_ones():
    w = I.Varlen("t", [300], 2, 64, seed=10)
    q, k, _ = w.tensors()
    v = torch.ones_like(q)
    out, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    assert np.abs(to_f64(out) - 1.0).max() <= 2.0 ** -8


# ---------------------------------------------------------------- invariants (bit-exact)

def test_varlen_equals_separate_runs_bitexact():
    lengths = [70, 1, 260, 129]
    w = I.Varlen("t", lengths, 4, 128, seed=11)
    q, k, v = w.tensors()
    out, kc, vc, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    for b, L in enumerate(lengths):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        o1, k1, v1, _ = run_varlen(q[s:e], k[s:e], v[s:e], [0, L], w.scale)
        np.testing.assert_array_equal(bits(o1), bits(out[s:e]))
        H, D = 4, 128
        np.testing.assert_array_equal(bits(k1), bits(kc)[s * H * D:e * H * D])


def test_sequences_and_heads_do_not_interfere():
    w = I.Varlen("t", [150, 90], 3, 64, seed=12)
    q, k, v = w.tensors()
    out, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    k2 = k.clone()
    k2[150:, 1] = -k2[150:, 1]
    out2, _, _, _ = run_varlen(q, k2, v, w.cu_seqlens, w.scale)
    a, b = bits(out), bits(out2)
    np.testing.assert_array_equal(a[:150], b[:150])
    np.testing.assert_array_equal(a[150:, 0], b[150:, 0])
    np.testing.assert_array_equal(a[150:, 2], b[150:, 2])
    assert not np.array_equal(a[151:, 1], b[151:, 1])


def test_deterministic():
    w = I.Varlen("t", [700, 3], 4, 128, seed=13)
    q, k, v = w.tensors()
    o1, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    o2, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    np.testing.assert_array_equal(bits(o1), bits(o2))


def test_max_seqlen_larger_than_needed():
    w = I.Varlen("t", [100, 20], 2, 32, seed=14)
    q, k, v = w.tensors()
    o1, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    o2, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale, max_seqlen=1000)
    np.testing.assert_array_equal(bits(o1), bits(o2))


def test_runs_on_caller_stream():
    w = I.Varlen("t", [333], 2, 128, seed=15)
    q, k, v = (t.cuda() for t in w.tensors())
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    outs = []
    for s in (torch.cuda.current_stream(), torch.cuda.Stream()):
        with torch.cuda.stream(s):
            out = torch.empty_like(q)
            kc = torch.empty_like(q)
            vc = torch.empty_like(q)
            P().prefill_attn_varlen(q, k, v, cu, kc, vc, out, scale=w.scale, max_seqlen=333)
        s.synchronize()
        outs.append(bits(out))
    np.testing.assert_array_equal(outs[0], outs[1])


# ---------------------------------------------------------------- chunked

def run_chunked(q, k, v, cu, pre, kc, vc, scale, max_seqlen=None):
    """kc, vc: device [B, H, cap, D] (modified in place); returns out (device)."""
    out = torch.empty_like(q, device="cuda")
    P().prefill_attn_chunked(q.cuda(), k.cuda(), v.cuda(),
                             torch.tensor(cu, dtype=torch.int32, device="cuda"), kc, vc, out,
                             torch.tensor(pre, dtype=torch.int32, device="cuda"), scale=scale,
                             max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("D", [32, 64, 128])
def test_chunked_small_full(D):
    """Chunks and decode rows with prefixes that are not tile multiples."""
    g = I.generator(200 + D)
    H = 3
    lengths = [1, 100, 1, 257, 64, 0, 1]
    prefix = [0, 37, 500, 129, 64, 10, 1]
    cap = 800
    cu = I.cu_from_lengths(lengths)
    N = cu[-1]
    q, k, v = (I.randn_bf16(g, (N, H, D)) for _ in range(3))
    kc0 = I.randn_bf16(g, (len(lengths), H, cap, D))
    vc0 = I.randn_bf16(g, (len(lengths), H, cap, D))
    # positions at and beyond the prefix hold the sentinel so stray writes show
    for b, p in enumerate(prefix):
        kc0[b, :, p:] = torch.tensor(SENTINEL, dtype=torch.int16).view(torch.bfloat16)
        vc0[b, :, p:] = torch.tensor(SENTINEL, dtype=torch.int16).view(torch.bfloat16)
    say("case chunked small D=%d" % D)
    kc, vc = kc0.cuda(), vc0.cuda()
    out = run_chunked(q, k, v, cu, prefix, kc, vc, I.default_scale(D))
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, prefix, kc0, vc0, I.default_scale(D))
    assert_close(out, ref, "chunked small D=%d" % D)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)


def test_chunked_equals_one_shot():
    """A prompt in 4 chunks of 256 through the cache reproduces the one-shot call
    (outputs to the parity bar: the work split differs, so the summation order
    does; cache bytes identical)."""
    T, C, H, D = 1024, 256, 4, 128
    w = I.Varlen("t", [T], H, D, seed=16)
    q, k, v = w.tensors()
    one, kc1, vc1, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    kc = torch.zeros((1, H, T, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    outs = []
    for c in range(T // C):
        sl = slice(c * C, (c + 1) * C)
        outs.append(run_chunked(q[sl], k[sl], v[sl], [0, C], [c * C], kc, vc, w.scale))
    assert_close(torch.cat(outs), to_f64(one), "chunked vs one-shot")
    np.testing.assert_array_equal(bits(kc).reshape(-1), bits(kc1))
    np.testing.assert_array_equal(bits(vc).reshape(-1), bits(vc1))


def test_decode_row_equals_prefill_row():
    H, D = 4, 128
    ps = [0, 1, 63, 64, 65, 200, 1000]
    T = max(ps) + 1
    w = I.Varlen("t", [T], H, D, seed=17)
    q, k, v = w.tensors()
    one, _, _, _ = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    B = len(ps)
    cap = T
    kc = torch.zeros((B, H, cap, D), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    for b, p in enumerate(ps):
        kc[b, :, :p] = k[:p].transpose(0, 1)
        vc[b, :, :p] = v[:p].transpose(0, 1)
    kcd, vcd = kc.cuda(), vc.cuda()
    out = run_chunked(q[ps], k[ps], v[ps], list(range(B + 1)), ps, kcd, vcd, w.scale)
    assert_close(out, to_f64(one)[ps], "decode vs prefill row")
    kb = bits(kcd)
    for b, p in enumerate(ps):
        np.testing.assert_array_equal(kb[b, :, p], bits(k)[p])


def test_chunked_workload_16_steps():
    """8192-token prompt in 512-token chunks beside 64 decode rows, all 16 steps."""
    wl = I.workload("chunked_8192x512_plus_64_decode_H32_D128")
    H, D, R = wl.num_heads, wl.head_dim, len(wl.contexts)
    say("case %s: drawing inputs" % "chunked_8192x512_plus_64_decode")
    t = wl.tensors()
    B = 1 + R
    kc = torch.zeros((B, H, wl.cap, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for r, ctx in enumerate(wl.contexts):
        kc[1 + r, :, :ctx] = t["pre_k"][r].cuda()
        vc[1 + r, :, :ctx] = t["pre_v"][r].cuda()
    rng = np.random.default_rng(0)
    for c in range(wl.num_chunks):
        st = wl.step(c)
        sl = slice(c * wl.chunk_len, (c + 1) * wl.chunk_len)
        q = torch.cat([t["pq"][sl], t["dq"]])
        k = torch.cat([t["pk"][sl], t["dk"]])
        v = torch.cat([t["pv"][sl], t["dv"]])
        kc_before = kc.cpu() if c in (0, 7, 15) else None
        vc_before = vc.cpu() if kc_before is not None else None
        say("  step %d" % c)
        out = run_chunked(q, k, v, st.cu_seqlens, st.prefix_lens, kc, vc, st.scale,
                          max_seqlen=wl.chunk_len)
        if kc_before is None:
            continue
        # sampled rows of the chunk (first, last, tile edges, random) + every decode row
        rows = sorted(set([0, 1, 63, 64, 127, 128, 255, 256, 511] +
                          rng.integers(0, 512, 24).tolist() + list(range(512, 512 + R))))
        ref = oracle.prefill_rows(q, k, v, st.cu_seqlens, st.scale, rows,
                                  prefix_lens=st.prefix_lens, k_cache=kc_before, v_cache=vc_before)
        assert_close(out[rows], ref, "chunk step %d" % c)
        kimg, vimg = oracle.cache_image(k, v, st.cu_seqlens, kc_before, vc_before,
                                        prefix_lens=st.prefix_lens)
        np.testing.assert_array_equal(bits(kc), kimg)
        np.testing.assert_array_equal(bits(vc), vimg)
    # after all chunks the prompt's cache holds exactly the prompt's K/V
    np.testing.assert_array_equal(bits(kc[0]), bits(t["pk"]).transpose(1, 0, 2))
    np.testing.assert_array_equal(bits(vc[0]), bits(t["pv"]).transpose(1, 0, 2))


def test_longmix_sampled():
    """Log-uniform lengths summing to 65536 plus one 32768-token sequence: every
    row of each sequence up to 2048 tokens, and of each longer one 256 evenly
    spaced rows plus the block and tile edges at its start and end; all heads;
    the whole cache bit for bit."""
    w = I.workload("longmix_65536_plus_32768_H32_D128")
    say("case %s: drawing inputs" % w.name)
    q, k, v = w.tensors()
    out, kc, vc, wholes = run_varlen(q, k, v, w.cu_seqlens, w.scale)
    rows = []
    for b, L in enumerate(w.lengths):
        s = w.cu_seqlens[b]
        if L <= 2048:
            rows += range(s, s + L)
            continue
        loc = [0, 1, 63, 64, 127, 128, 129, L // 2, L - 129, L - 128, L - 65, L - 64, L - 2, L - 1]
        loc += list(np.linspace(0, L - 1, 256).astype(int))
        rows += sorted(set(s + x for x in loc if 0 <= x < L))
    say("  oracle on %d sampled rows (about half a minute)" % len(rows))
    ref = oracle.prefill_rows(q, k, v, w.cu_seqlens, w.scale, rows)
    assert_close(out[rows], ref, w.name)
    n = w.num_tokens * w.num_heads * w.head_dim
    sent = np.full(n, SENTINEL, np.uint16)
    kimg, vimg = oracle.cache_image(k, v, w.cu_seqlens, sent, sent)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)
    assert all(guards_intact(x) for x in wholes)


def test_offsets_beyond_4gib():
    """640 sequences of 1024 tokens, 32 query heads over 8 K/V heads: q and out
    span 5.4 GB, so the last sequences' rows sit beyond every 32-bit byte
    offset.  Inputs are drawn on the device from a seeded generator; three
    sequences (first, middle, last) are copied back and checked against the
    oracle on sampled rows, with their whole cache blocks bit for bit."""
    B, T, H, HK, D = 640, 1024, 32, 8, 128
    N = B * T
    g = torch.Generator(device="cuda").manual_seed(1300)

    def draw(shape):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    say("case offsets beyond 4 GiB: drawing %d tokens on the device" % N)
    q, k, v = draw((N, H, D)), draw((N, HK, D)), draw((N, HK, D))
    cu = torch.arange(0, N + 1, T, dtype=torch.int32, device="cuda")
    kc = torch.empty(N * HK * D, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.empty_like(q)
    scale = I.default_scale(D)
    P().prefill_attn_varlen(q, k, v, cu, kc, vc, out, scale=scale, max_seqlen=T)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 127, 128, 511, 1000, 1022, 1023]
    for b in (0, B // 2, B - 1):
        s = b * T
        qs, ks, vs = q[s:s + T].cpu(), k[s:s + T].cpu(), v[s:s + T].cpu()
        ref = oracle.prefill_rows(qs, ks, vs, [0, T], scale, rows)
        assert_close(out[s:s + T][rows], ref, "sequence %d (out byte offset %d)" % (b, s * H * D * 2))
        z = np.zeros(T * HK * D, np.uint16)
        kimg, vimg = oracle.cache_image(ks, vs, [0, T], z, z)
        blk = slice(s * HK * D, (s + T) * HK * D)
        np.testing.assert_array_equal(bits(kc[blk]), kimg, err_msg="k cache of sequence %d" % b)
        np.testing.assert_array_equal(bits(vc[blk]), vimg, err_msg="v cache of sequence %d" % b)
    del q, k, v, kc, vc, out


# ---------------------------------------------------------------- check mode

def test_check_mode_rejects_bad_metadata():
    mod = P()
    w = I.Varlen("t", [10, 10], 2, 64, seed=18)
    q, k, v = (t.cuda() for t in w.tensors())
    out, kc, vc = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    prev = mod.pa_set_check_mode(True)
    try:
        bad = torch.tensor([0, 12, 20], dtype=torch.int32, device="cuda")  # length 12 > 10
        with pytest.raises(mod.PrefillAttnError, match="SEQLENS"):
            mod.prefill_attn_varlen(q, k, v, bad, kc, vc, out, max_seqlen=10)
        bad = torch.tensor([1, 10, 20], dtype=torch.int32, device="cuda")
        with pytest.raises(mod.PrefillAttnError, match="SEQLENS"):
            mod.prefill_attn_varlen(q, k, v, bad, kc, vc, out, max_seqlen=10)
        cu = torch.tensor([0, 10, 20], dtype=torch.int32, device="cuda")
        kc4 = torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
        vc4 = torch.zeros_like(kc4)
        pre = torch.tensor([0, 7], dtype=torch.int32, device="cuda")  # 7 + 10 > 16
        with pytest.raises(mod.PrefillAttnError, match="CAPACITY"):
            mod.prefill_attn_chunked(q, k, v, cu, kc4, vc4, out, pre, max_seqlen=10)
        pre = torch.tensor([0, 6], dtype=torch.int32, device="cuda")
        mod.prefill_attn_chunked(q, k, v, cu, kc4, vc4, out, pre, max_seqlen=10)
        torch.cuda.synchronize()
    finally:
        mod.pa_set_check_mode(prev)
