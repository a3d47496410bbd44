"""Pins for the float64 oracle: checks against things other than itself.

Each test fixes the oracle to something the pages or the mathematics fix:
brute force with a materialised mask (tests/bruteforce.py), torch's float64
scaled_dot_product_attention as a library routine, closed forms (running
means), invariants (row sums, isolation of requests and heads, chunked equals
one-shot, decode row equals prefill row) and the cache-size figures the pages
print (tests/golden/pages_worked_examples.json).  A dropped term, a wrong sign,
a transposed operand or a shifted index in oracle.c fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests import bruteforce as BF

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "pages_worked_examples.json")))


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_varlen(lengths, H, D, seed):
    w = I.Varlen("t", lengths, H, D, seed=seed)
    q, k, v = w.tensors()
    return w, bits(q), bits(k), bits(v)


def f64(b):
    return BF.bf16_to_f64(b)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("lengths,H,D,seed", [
    ([3], 4, 32, 11),            # toy: 3 tokens, 4 heads, head_dim 32
    ([64], 4, 32, 1),            # single T=64 workload
    ([5, 2, 3], 2, 32, 12),      # cu_seqlens [0,5,7,10]
    ([1, 17, 0, 40], 3, 64, 13),  # includes an empty sequence
])
def test_matches_bruteforce(lengths, H, D, seed):
    w, q, k, v = rand_varlen(lengths, H, D, seed)
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    ref = BF.varlen(q, k, v, w.cu_seqlens, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_matches_torch_sdpa_float64():
    """A library routine: torch's float64 CPU attention with is_causal."""
    w, q, k, v = rand_varlen([96], 4, 128, 21)
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    Q = torch.from_numpy(f64(q)).permute(1, 0, 2)
    K = torch.from_numpy(f64(k)).permute(1, 0, 2)
    V = torch.from_numpy(f64(v)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, is_causal=True, scale=w.scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_chunked_matches_torch_sdpa_with_prefix_mask():
    """Bottom-right alignment: query i at absolute prefix+i sees keys 0..prefix+i."""
    H, D, pre, n, cap = 2, 64, 37, 20, 64
    g = I.generator(31)
    q = I.randn_bf16(g, (n, H, D))
    k = I.randn_bf16(g, (n, H, D))
    v = I.randn_bf16(g, (n, H, D))
    kc = I.randn_bf16(g, (1, H, cap, D))
    vc = I.randn_bf16(g, (1, H, cap, D))
    scale = I.default_scale(D)
    out, kimg, vimg, _ = oracle.prefill_chunked(bits(q), bits(k), bits(v), [0, n], [pre],
                                                bits(kc), bits(vc), scale)
    Kall = torch.cat([kc[0, :, :pre].double(), k.double().permute(1, 0, 2)], dim=1)
    Vall = torch.cat([vc[0, :, :pre].double(), v.double().permute(1, 0, 2)], dim=1)
    mask = torch.arange(pre + n)[None, :] <= (pre + torch.arange(n))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double().permute(1, 0, 2), Kall, Vall, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    # own K/V appended at prefix..prefix+n-1, nothing else touched
    np.testing.assert_array_equal(kimg[0, :, pre:pre + n], bits(k).transpose(1, 0, 2))
    np.testing.assert_array_equal(vimg[0, :, pre:pre + n], bits(v).transpose(1, 0, 2))
    np.testing.assert_array_equal(kimg[0, :, :pre], bits(kc)[0, :, :pre])
    np.testing.assert_array_equal(kimg[0, :, pre + n:], bits(kc)[0, :, pre + n:])
    np.testing.assert_array_equal(vimg[0, :, pre + n:], bits(vc)[0, :, pre + n:])


# ---------------------------------------------------------------- closed forms

def test_first_row_and_length_one_return_own_v_exactly():
    w, q, k, v = rand_varlen([1, 9, 1, 33], 4, 32, 41)
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    for b in range(len(w.lengths)):
        s = w.cu_seqlens[b]
        np.testing.assert_array_equal(out[s], f64(v)[s])


def test_v_ones_gives_ones_and_rows_sum_to_one():
    w, q, k, v = rand_varlen([50], 3, 32, 42)
    ones = bits(torch.ones(50, 3, 32, dtype=torch.bfloat16))
    out, _, _, probs = oracle.prefill_varlen(q, k, ones, w.cu_seqlens, w.scale, want_probs=True)
    np.testing.assert_array_equal(out, np.ones_like(out))
    np.testing.assert_allclose(probs.sum(axis=2), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", ["identical_keys", "zero_scale"])
def test_running_mean_closed_form(mode):
    """All scores of a row equal -> weights uniform over keys 0..i -> causal running mean of V."""
    w, q, k, v = rand_varlen([7, 60], 2, 64, 43)
    scale = w.scale
    if mode == "identical_keys":
        k = np.broadcast_to(k[:1], k.shape).copy()  # one key for every position
        for b in range(2):
            s = w.cu_seqlens[b]
            k[s:w.cu_seqlens[b + 1]] = k[s]
    else:
        scale = 0.0
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, scale)
    V = f64(v)
    for b in range(2):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        mean = np.cumsum(V[s:e], axis=0) / np.arange(1, e - s + 1)[:, None, None]
        np.testing.assert_allclose(out[s:e], mean, rtol=1e-13, atol=1e-14)


def test_chunked_running_mean_counts_prefix():
    """scale 0 in a chunk with prefix p: out_i = mean of prefix V and own V_0..i."""
    H, D, pre, n, cap = 2, 32, 10, 6, 16
    g = I.generator(44)
    q, k, v = (I.randn_bf16(g, (n, H, D)) for _ in range(3))
    kc = I.randn_bf16(g, (1, H, cap, D))
    vc = I.randn_bf16(g, (1, H, cap, D))
    out, _, _, _ = oracle.prefill_chunked(bits(q), bits(k), bits(v), [0, n], [pre],
                                          bits(kc), bits(vc), 0.0)
    Vall = np.concatenate([f64(bits(vc))[0, :, :pre], f64(bits(v)).transpose(1, 0, 2)], axis=1)
    for i in range(n):
        np.testing.assert_allclose(out[i], Vall[:, :pre + i + 1].mean(axis=1),
                                   rtol=1e-13, atol=1e-14)


def test_one_hot_v_exposes_probabilities():
    """V[j] = e_j (T <= D): out[i, j] = P[i, j]; zero above the diagonal, rows sum to 1."""
    T, H, D = 24, 2, 32
    w, q, k, _ = rand_varlen([T], H, D, 45)
    eye = np.zeros((T, H, D), dtype=np.float32)
    for j in range(T):
        eye[j, :, j] = 1.0
    v = bits(torch.from_numpy(eye).to(torch.bfloat16))
    out, _, _, probs = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale, want_probs=True)
    for h in range(H):
        P = out[:, h, :T]
        assert np.all(np.triu(P, 1) == 0.0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
        _, pref = BF.attention_one(f64(q)[:, h], f64(k)[:, h], f64(v)[:, h], w.scale)
        np.testing.assert_allclose(P, pref, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(probs[h], pref, rtol=1e-12, atol=1e-15)


def test_two_keys_logistic_form():
    """Row 1 of a 2-token sequence: weight on key 1 is the logistic of the score gap."""
    w, q, k, v = rand_varlen([2], 1, 32, 46)
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    Q, K, V = f64(q)[:, 0], f64(k)[:, 0], f64(v)[:, 0]
    gap = w.scale * (float(np.dot(Q[1], K[1])) - float(np.dot(Q[1], K[0])))
    a = 1.0 / (1.0 + np.exp(-gap))
    np.testing.assert_allclose(out[1, 0], (1 - a) * V[0] + a * V[1], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_varlen_equals_separate_runs_exactly():
    w, q, k, v = rand_varlen([5, 2, 3], 4, 32, 47)
    assert w.cu_seqlens == GOLDEN["varlen_metadata"]["cu_seqlens"]
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    for b in range(3):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        sep, _, _, _ = oracle.prefill_varlen(q[s:e], k[s:e], v[s:e], [0, e - s], w.scale)
        np.testing.assert_array_equal(out[s:e], sep)


def test_requests_and_heads_do_not_interfere():
    w, q, k, v = rand_varlen([12, 20], 3, 32, 48)
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    k2 = k.copy()
    k2[12:, 1] ^= 0x0101  # perturb sequence 1, head 1
    out2, _, _, _ = oracle.prefill_varlen(q, k2, v, w.cu_seqlens, w.scale)
    np.testing.assert_array_equal(out2[:12], out[:12])
    np.testing.assert_array_equal(out2[12:, 0], out[12:, 0])
    np.testing.assert_array_equal(out2[12:, 2], out[12:, 2])
    assert not np.array_equal(out2[13:, 1], out[13:, 1])


def test_chunked_equals_one_shot():
    """A prompt processed in chunks through the cache reproduces the one-shot call."""
    T, C, H, D = 96, 32, 2, 32
    w, q, k, v = rand_varlen([T], H, D, 49)
    one, kimg1, vimg1, _ = oracle.prefill_varlen(
        q, k, v, w.cu_seqlens, w.scale,
        k_cache=np.zeros(T * H * D, np.uint16), v_cache=np.zeros(T * H * D, np.uint16))
    kc = np.zeros((1, H, T, D), np.uint16)
    vc = np.zeros((1, H, T, D), np.uint16)
    outs = []
    for c in range(T // C):
        sl = slice(c * C, (c + 1) * C)
        o, kc, vc, _ = oracle.prefill_chunked(q[sl], k[sl], v[sl], [0, C], [c * C], kc, vc, w.scale)
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs), one, rtol=1e-12, atol=1e-14)
    # [1, H, cap=T, D] chunked layout is byte-identical to the varlen [H, T, D] block
    np.testing.assert_array_equal(kc.reshape(-1), kimg1)
    np.testing.assert_array_equal(vc.reshape(-1), vimg1)


def test_decode_row_equals_prefill_row():
    """A length-1 row with prefix p equals row p of a prefill over the same p+1 tokens."""
    p, H, D = 30, 2, 32
    w, q, k, v = rand_varlen([p + 1], H, D, 50)
    one, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    kc = np.zeros((1, H, p + 8, D), np.uint16)
    vc = np.zeros((1, H, p + 8, D), np.uint16)
    kc[0, :, :p] = k[:p].transpose(1, 0, 2)
    vc[0, :, :p] = v[:p].transpose(1, 0, 2)
    o, kimg, vimg, _ = oracle.prefill_chunked(q[p:], k[p:], v[p:], [0, 1], [p], kc, vc, w.scale)
    np.testing.assert_allclose(o[0], one[p], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(kimg[0, :, p], k[p])
    np.testing.assert_array_equal(vimg[0, :, p], v[p])


def test_sampled_rows_equal_full_run():
    w, q, k, v = rand_varlen([33, 1, 70], 2, 64, 51)
    out, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    rows = [0, 32, 33, 34, 60, 103]
    sub = oracle.prefill_rows(q, k, v, w.cu_seqlens, w.scale, rows)
    np.testing.assert_array_equal(sub, out[rows])


def test_sampled_rows_chunked_equal_full_run():
    H, D, cap = 2, 32, 40
    g = I.generator(52)
    n = [5, 1, 1]
    pre = [12, 30, 0]
    N = sum(n)
    q, k, v = (I.randn_bf16(g, (N, H, D)) for _ in range(3))
    kc = I.randn_bf16(g, (3, H, cap, D))
    vc = I.randn_bf16(g, (3, H, cap, D))
    cu = I.cu_from_lengths(n)
    out, _, _, _ = oracle.prefill_chunked(bits(q), bits(k), bits(v), cu, pre, bits(kc), bits(vc), 0.3)
    sub = oracle.prefill_rows(bits(q), bits(k), bits(v), cu, 0.3, list(range(N)),
                              prefix_lens=pre, k_cache=bits(kc), v_cache=bits(vc))
    np.testing.assert_array_equal(sub, out)


def test_thread_count_does_not_change_result():
    w, q, k, v = rand_varlen([40, 23], 4, 32, 53)
    a, _, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    b = np.zeros_like(a)
    for h in range(4):  # one head at a time: a different work split
        bh, _, _, _ = oracle.prefill_varlen(q[:, h:h + 1].copy(), k[:, h:h + 1].copy(),
                                            v[:, h:h + 1].copy(), w.cu_seqlens, w.scale)
        b[:, h] = bh[:, 0]
    np.testing.assert_array_equal(a, b)


def test_rejects_bad_metadata():
    w, q, k, v = rand_varlen([4, 4], 1, 32, 54)
    with pytest.raises(ValueError):
        oracle.prefill_varlen(q, k, v, [0, 5, 3, 8], w.scale)  # cu not monotonic
    with pytest.raises(ValueError):
        oracle.prefill_chunked(q, k, v, [0, 4, 8], [0, 6], np.zeros((2, 1, 8, 32), np.uint16),
                               np.zeros((2, 1, 8, 32), np.uint16), w.scale)  # 6 + 4 > cap 8


# ---------------------------------------------------------------- the pages' figures

def test_cache_bytes_match_pages_T512():
    """Per-layer K+V bytes for 32 heads x 512 tokens x 128 in bf16 (printed on the pages)."""
    fx = GOLDEN["kv_bytes_per_layer_T512"]
    T, H, D = fx["seq_len"], fx["num_heads"], fx["head_dim"]
    w, q, k, v = rand_varlen([T], H, D, 55)
    sentinel = np.full(T * H * D + 64, 0x7FC1, np.uint16)  # bf16 NaN pattern, extra guard
    _, kimg, vimg, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale,
                                             k_cache=sentinel, v_cache=sentinel)
    written = (np.count_nonzero(kimg != sentinel) + np.count_nonzero(vimg != sentinel))
    # every element of k/v is copied once; N(0,1) bf16 never equals the sentinel bits
    assert written * fx["bytes_per_element"] == fx["bytes"]
    assert np.all(kimg[T * H * D:] == 0x7FC1)
    # head-major: element (h, t, d) of the image is k[t, h, d]
    np.testing.assert_array_equal(kimg[:T * H * D].reshape(H, T, D), k.transpose(1, 0, 2))


def test_cache_bytes_closed_forms_from_pages():
    fx = GOLDEN["kv_bytes_per_layer_T4096"]
    b = 2 * fx["num_heads"] * fx["seq_len"] * fx["head_dim"] * fx["bytes_per_element"]
    assert b == fx["approx_mib"] * 2 ** 20
    fx = GOLDEN["kv_bytes_per_token_model"]
    per_layer = 2 * fx["num_heads"] * fx["head_dim"] * fx["bytes_per_element"]
    assert per_layer * fx["num_layers"] == fx["bytes"]
    assert per_layer == 16384
    fx = GOLDEN["score_matrix_bytes_T8192"]
    assert fx["seq_len"] ** 2 * fx["bytes_per_element"] == fx["approx_mib"] * 2 ** 20


def test_toy_shapes_from_pages():
    """3 tokens, 4 heads of 32: the layer's K cache is [4, 3, 32]; decode grows it to 4."""
    fx = GOLDEN["toy_prefill_shapes"]
    T, H, D = fx["tokens"], fx["num_heads"], fx["head_dim"]
    assert H * D == fx["hidden"]
    w, q, k, v = rand_varlen([T], H, D, 56)
    _, kimg, _, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale,
                                          k_cache=np.zeros(T * H * D, np.uint16),
                                          v_cache=np.zeros(T * H * D, np.uint16))
    assert list(kimg.reshape(H, T, D).shape) == fx["k_cache_layer_shape"]
    dg = GOLDEN["toy_decode_growth"]
    kc = np.zeros((1, H, dg["cache_len_after"], D), np.uint16)
    vc = np.zeros_like(kc)
    kc[0, :, :T] = k.transpose(1, 0, 2)
    vc[0, :, :T] = v.transpose(1, 0, 2)
    g = I.generator(57)
    nq, nk, nv = (bits(I.randn_bf16(g, (1, H, D))) for _ in range(3))
    _, _, _, probs = oracle.prefill_chunked(nq, nk, nv, [0, 1], [dg["cache_len_before"]],
                                            kc, vc, w.scale, want_probs=True)
    assert probs.shape == (H, 1, dg["cache_len_after"])  # scores over 3 cached + itself


def test_decode_token_sees_prefix_and_itself():
    fx = GOLDEN["decode_visible_positions"]
    p, H, D = fx["prompt_tokens"], 1, 32
    g = I.generator(58)
    kc = bits(I.randn_bf16(g, (1, H, p + 1, D)))
    vc = bits(I.randn_bf16(g, (1, H, p + 1, D)))
    q, k, v = (bits(I.randn_bf16(g, (1, H, D))) for _ in range(3))
    _, _, _, probs = oracle.prefill_chunked(q, k, v, [0, 1], [p], kc, vc, 0.2, want_probs=True)
    assert probs.shape[2] == fx["positions_attended_by_next_token"]
    assert np.all(probs > 0)


def test_causal_pair_count():
    """Non-zero weights of a T-token row block = T(T+1)/2 causal pairs (half the full square)."""
    T = 48
    w, q, k, v = rand_varlen([T], 1, 32, 59)
    _, _, _, probs = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale, want_probs=True)
    assert np.count_nonzero(probs) == T * (T + 1) // 2


def test_cache_image_only_matches_full_oracle():
    w, q, k, v = rand_varlen([7, 1, 30], 2, 32, 60)
    sent = np.full(w.num_tokens * 2 * 32 + 16, 0x7FC1, np.uint16)
    _, kimg, vimg, _ = oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale,
                                             k_cache=sent, v_cache=sent)
    kc, vc = oracle.cache_image(k, v, w.cu_seqlens, sent, sent)
    np.testing.assert_array_equal(kc, kimg)
    np.testing.assert_array_equal(vc, vimg)
    g = I.generator(61)
    n, pre = [4, 1], [9, 3]
    cu = I.cu_from_lengths(n)
    kq, kk, kv = (bits(I.randn_bf16(g, (5, 2, 32))) for _ in range(3))
    kc0 = bits(I.randn_bf16(g, (2, 2, 16, 32)))
    vc0 = bits(I.randn_bf16(g, (2, 2, 16, 32)))
    _, kimg, vimg, _ = oracle.prefill_chunked(kq, kk, kv, cu, pre, kc0, vc0, 0.1)
    kc, vc = oracle.cache_image(kk, kv, cu, kc0, vc0, prefix_lens=pre)
    np.testing.assert_array_equal(kc, kimg)
    np.testing.assert_array_equal(vc, vimg)


# ---------------------------------------------------------------- grouped K/V heads [P5 §2.4]

def _gqa_inputs(n, H, HK, D, seed):
    g = I.generator(seed)
    q = I.randn_bf16(g, (n, H, D))
    k = I.randn_bf16(g, (n, HK, D))
    v = I.randn_bf16(g, (n, HK, D))
    return q, k, v


@pytest.mark.parametrize("H,HK", [(8, 2), (6, 3), (4, 1)])
def test_gqa_matches_torch_sdpa_enable_gqa(H, HK):
    """A library routine: torch's float64 attention with enable_gqa (each K/V
    head serves H/HK consecutive query heads); HK = 1 is multi-query."""
    n, D = 70, 64
    q, k, v = _gqa_inputs(n, H, HK, D, 300 + H * 10 + HK)
    scale = I.default_scale(D)
    out, _, _, _ = oracle.prefill_varlen(bits(q), bits(k), bits(v), [0, n], scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double().permute(1, 0, 2), k.double().permute(1, 0, 2), v.double().permute(1, 0, 2),
        is_causal=True, scale=scale, enable_gqa=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_gqa_equals_mha_on_repeated_heads():
    """Grouping is the plain repetition of each K/V head over its query heads."""
    n, H, HK, D = 41, 8, 2, 32
    q, k, v = _gqa_inputs(n, H, HK, D, 331)
    scale = I.default_scale(D)
    out, _, _, _ = oracle.prefill_varlen(bits(q), bits(k), bits(v), [0, 17, n], scale)
    kr = k.repeat_interleave(H // HK, dim=1)
    vr = v.repeat_interleave(H // HK, dim=1)
    ref, _, _, _ = oracle.prefill_varlen(bits(q), bits(kr), bits(vr), [0, 17, n], scale)
    np.testing.assert_array_equal(out, ref)


def test_gqa_chunked_matches_torch_sdpa_with_prefix_mask():
    H, HK, D, pre, n, cap = 6, 2, 64, 29, 13, 48
    q, k, v = _gqa_inputs(n, H, HK, D, 341)
    g = I.generator(342)
    kc = I.randn_bf16(g, (1, HK, cap, D))
    vc = I.randn_bf16(g, (1, HK, cap, D))
    scale = I.default_scale(D)
    out, kimg, vimg, _ = oracle.prefill_chunked(bits(q), bits(k), bits(v), [0, n], [pre],
                                                bits(kc), bits(vc), scale)
    Kall = torch.cat([kc[0, :, :pre].double(), k.double().permute(1, 0, 2)], dim=1)
    Vall = torch.cat([vc[0, :, :pre].double(), v.double().permute(1, 0, 2)], dim=1)
    mask = torch.arange(pre + n)[None, :] <= (pre + torch.arange(n))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double().permute(1, 0, 2), Kall, Vall, attn_mask=mask, scale=scale, enable_gqa=True)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(kimg[0, :, pre:pre + n], bits(k).transpose(1, 0, 2))
    np.testing.assert_array_equal(vimg[0, :, pre:pre + n], bits(v).transpose(1, 0, 2))
    np.testing.assert_array_equal(kimg[0, :, :pre], bits(kc)[0, :, :pre])


def test_gqa_varlen_cache_holds_kv_heads_only():
    """The cache keeps one row per K/V head: sequence b's block is [HK, len_b, D]."""
    H, HK, D = 8, 2, 32
    lengths = [5, 11]
    q, k, v = _gqa_inputs(sum(lengths), H, HK, D, 351)
    cu = I.cu_from_lengths(lengths)
    fill = np.full(sum(lengths) * HK * D, 0x7FC1, np.uint16)
    _, kimg, vimg, _ = oracle.prefill_varlen(bits(q), bits(k), bits(v), cu, 0.125,
                                             k_cache=fill, v_cache=fill)
    for b, L in enumerate(lengths):
        blk = kimg[cu[b] * HK * D:(cu[b] + L) * HK * D].reshape(HK, L, D)
        np.testing.assert_array_equal(blk, bits(k)[cu[b]:cu[b] + L].transpose(1, 0, 2))
        blk = vimg[cu[b] * HK * D:(cu[b] + L) * HK * D].reshape(HK, L, D)
        np.testing.assert_array_equal(blk, bits(v)[cu[b]:cu[b] + L].transpose(1, 0, 2))


def test_gqa_rejects_heads_that_do_not_divide():
    q, k, v = _gqa_inputs(4, 6, 4, 32, 361)
    with pytest.raises(ValueError):
        oracle.prefill_varlen(bits(q), bits(k), bits(v), [0, 4], 0.1)


# ---------------------------------------------------------------- INT8 KV rows
# Quantised cache rows ("大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.3:
# K and V only, INT8 halves the cache, per-token scales are one of the listed
# granularities).  The oracle's reading: symmetric, one float32 scale per
# (token, K/V head) row, scale = amax/127, code = rint(x * 127/amax).

def _bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)


def test_int8_exact_grid_ties_to_even():
    """amax = 127/64 makes 127/amax = 64 exactly, so every code is
    round-half-even(64 x) of an exact product: checked with Fractions.  The
    other entries are k/128, so odd k land exactly on a tie."""
    from fractions import Fraction
    ks = [-127, 5, -5, 7, 3, -3, 1, 0, 64, 65, -66, 100, 2, 9, -11]
    x = _bf16([127 / 64.0] + [k / 128.0 for k in ks])
    codes, scales = oracle.quantize_rows_int8(x.view(1, -1))
    want = [127] + [round(Fraction(64) * Fraction(k, 128)) for k in ks]  # Python round: ties to even
    assert codes[0].tolist() == want
    assert want[2:5] == [2, -2, 4] and want[5:7] == [2, -2]  # 2.5->2, -2.5->-2, 3.5->4, 1.5->2
    assert scales[0] == np.float32(1 / 64)


def test_int8_hand_example():
    """Row [1, -2, 0.5, 0.25, 0.75, -1.5, 0, 0]: amax 2, 127/amax = 63.5 exactly,
    products exact, codes 64 (63.5 to even), -127, 32 (31.75), 16 (15.875),
    48 (47.625), -95 (-95.25), 0, 0; scale = 2/127 rounded to float32."""
    from fractions import Fraction
    codes, scales = oracle.quantize_rows_int8(_bf16([[1, -2, 0.5, 0.25, 0.75, -1.5, 0, 0]]))
    assert codes[0].tolist() == [64, -127, 32, 16, 48, -95, 0, 0]
    s = Fraction(float(scales[0]))
    ulp = Fraction(2) ** (-7 - 23)  # 2/127 lies in [2^-7, 2^-6)
    assert abs(s - Fraction(2, 127)) <= ulp / 2


@pytest.mark.parametrize("sigma", [1.0, 1e-3, 40.0])
def test_int8_properties_random_rows(sigma):
    g = torch.Generator().manual_seed(77)
    x = (torch.randn(500, 128, generator=g) * sigma).to(torch.bfloat16)
    codes, scales = oracle.quantize_rows_int8(x)
    xf = x.float().double().numpy()
    c = codes.astype(np.float64)
    s = scales.astype(np.float64)
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    # the largest |x| of each row maps to +-127 with the sign of x
    arg = np.abs(xf).argmax(axis=1)
    top = c[np.arange(len(arg)), arg]
    assert np.all(np.abs(top) == 127) and np.all(np.sign(top) == np.sign(xf[np.arange(len(arg)), arg]))
    # dequantisation error at most half a step (plus float32 rounding slop)
    err = np.abs(xf - c * s[:, None])
    assert np.all(err <= 0.5 * s[:, None] * (1 + 2.0 ** -20) + 2.0 ** -22 * np.abs(xf))
    # scale is amax / 127 to float32 accuracy
    amax = np.abs(xf).max(axis=1)
    assert np.allclose(s, amax / 127, rtol=2.0 ** -23, atol=0)
    # odd symmetry and invariance under power-of-two scaling
    cn, sn = oracle.quantize_rows_int8(-x)
    assert np.array_equal(cn, -codes) and np.array_equal(sn, scales)
    c4, s4 = oracle.quantize_rows_int8((x.float() * 4).to(torch.bfloat16))
    assert np.array_equal(c4, codes) and np.array_equal(s4, scales * 4)


def test_int8_zero_and_tiny_rows():
    x = torch.zeros(3, 64, dtype=torch.bfloat16)
    x[1, 5] = 1e-35   # amax below 2^-100: stored as zeros
    x[2, 7] = -3.0
    codes, scales = oracle.quantize_rows_int8(x)
    assert scales[0] == 0 and scales[1] == 0 and not codes[:2].any()
    assert codes[2, 7] == -127 and np.count_nonzero(codes[2]) == 1
    from fractions import Fraction
    assert abs(Fraction(float(scales[2])) - Fraction(3, 127)) <= Fraction(2) ** (-6 - 23) / 2


def test_int8_cache_image_layout_bruteforce():
    """Sequence b's [HK, len_b, D] block at row cu[b]*HK: placement checked
    row by row against single-row quantisation."""
    lengths, HK, D = [3, 1, 5], 2, 32
    g = torch.Generator().manual_seed(78)
    N = sum(lengths)
    k = torch.randn(N, HK, D, generator=g).to(torch.bfloat16)
    v = torch.randn(N, HK, D, generator=g).to(torch.bfloat16)
    cu = [0, 3, 4, 9]
    kq, ks, vq, vs = oracle.cache_image_int8(k, v, cu)
    assert kq.shape == (N * HK * D,) and ks.shape == (N * HK,)
    for b, L in enumerate(lengths):
        for hk in range(HK):
            for t in range(L):
                row = cu[b] * HK + hk * L + t
                ck, sk = oracle.quantize_rows_int8(k[cu[b] + t, hk].view(1, D))
                cv, sv = oracle.quantize_rows_int8(v[cu[b] + t, hk].view(1, D))
                assert np.array_equal(kq[row * D:(row + 1) * D], ck[0]) and ks[row] == sk[0]
                assert np.array_equal(vq[row * D:(row + 1) * D], cv[0]) and vs[row] == sv[0]


# ---------------------------------------------------------------- FP8 rows
# FP8 cache rows ("大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.3
# lists low-precision cache formats; the encoding is the OCP 8-bit E4M3 format
# by reading): sign, 4 exponent bits with bias 7, 3 mantissa bits,
# subnormals m/8 * 2^-6, no infinities, S.1111.111 NaN, largest finite 448.

def test_e4m3_textbook_values():
    """Code values fixed by the format definition."""
    D = oracle.e4m3_decode
    assert D(0x00) == 0.0 and np.signbit(D(0x80)) and D(0x80) == 0.0
    assert D(0x38) == 1.0 and D(0xB8) == -1.0
    assert D(0x7E) == 448.0 and D(0xFE) == -448.0
    assert D(0x3F) == 1.875 and D(0x40) == 2.0 and D(0x30) == 0.5
    assert D(0x08) == 2.0 ** -6 and D(0x01) == 2.0 ** -9 and D(0x07) == 7 * 2.0 ** -9
    assert np.isnan(D(0x7F)) and np.isnan(D(0xFF))
    # 126 finite positive magnitudes, strictly increasing with the code
    vals = [D(c) for c in range(0x00, 0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_e4m3_every_code_round_trips():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


def test_e4m3_midpoints_round_to_even():
    """Between neighbouring codes: the exact midpoint goes to the code with an
    even mantissa, anything off it to the nearer code (both signs)."""
    D, E = oracle.e4m3_decode, oracle.e4m3_encode
    for c in range(0x00, 0x7E):
        lo, hi = D(c), D(c + 1)
        mid = (lo + hi) / 2  # exact in float32: at most five significant bits
        assert np.float32(mid) == mid
        even = c if c % 2 == 0 else c + 1
        assert E(mid) == even and E(-mid) == even | 0x80, hex(c)
        assert E(np.nextafter(np.float32(mid), np.float32(0))) == c
        assert E(np.nextafter(np.float32(mid), np.float32(1e30))) == c + 1


def test_e4m3_beyond_the_largest_value():
    """448 is the largest finite value: the midpoint 464 rounds to it (even
    mantissa), anything that would round past it is NaN (no infinities).  The
    row quantiser never produces such values (|x| * 448 / amax <= 448 up to
    float32 rounding)."""
    E = oracle.e4m3_encode
    assert E(448.0) == 0x7E and E(460.0) == 0x7E and E(464.0) == 0x7E
    assert E(np.nextafter(np.float32(464.0), np.float32(1e30))) == 0x7F
    assert E(-500.0) == 0xFF and E(1e30) == 0x7F


def test_fp8_row_hand_example():
    """amax = 448: scale 1 and every code is the E4M3 rounding of x itself."""
    x = _bf16([[448, -1, 0.3, 1.0625, 1.1875, 2.0 ** -10, -3 * 2.0 ** -10, 0]])
    codes, scales = oracle.quantize_rows_fp8(x)
    assert scales.tolist() == [1.0]
    assert codes[0].tolist() == [0x7E, 0xB8, 0x2A, 0x38, 0x3A, 0x00, 0x82, 0x00]


@pytest.mark.parametrize("sigma", [1e-3, 1.0, 300.0])
def test_fp8_properties_random_rows(sigma):
    g = torch.Generator().manual_seed(91)
    x = (torch.randn(64, 128, generator=g) * sigma).to(torch.bfloat16)
    codes, scales = oracle.quantize_rows_fp8(x)
    xf = x.double().numpy()
    amax = np.abs(xf).max(axis=1)
    assert np.array_equal(scales, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    dec = np.vectorize(oracle.e4m3_decode)(codes.astype(np.int64))
    assert np.all(np.isfinite(dec))
    # error: half a mantissa step (2^-4 relative) for normals, half the
    # subnormal step 2^-10 in code units otherwise, plus float32 rounding
    y = xf * (448.0 / amax[:, None])
    err = np.abs(dec - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 2.0 ** -20) + np.abs(y) * 2.0 ** -22)
    # each row's largest |x| encodes as +-448
    top = codes[np.arange(64), np.abs(xf).argmax(axis=1)]
    assert np.all((top & 0x7F) == 0x7E)
    # odd symmetry: -x flips exactly the sign bits
    cn, sn = oracle.quantize_rows_fp8(-x)
    assert np.array_equal(sn, scales) and np.array_equal(cn, codes ^ 0x80)


def test_fp8_zero_and_tiny_rows():
    x = torch.zeros(3, 16, dtype=torch.bfloat16)
    x[1, 3] = 1e-35
    x[2, :] = -2.0 ** -110
    codes, scales = oracle.quantize_rows_fp8(x)
    assert scales.tolist() == [0.0, 0.0, 0.0]
    assert np.all(codes[0] == 0) and np.all(codes[1] == 0)
    assert np.all(codes[2] == 0x80)  # x * 0 keeps the sign


def test_fp8_cache_image_layout_bruteforce():
    lengths, HK, D = [3, 1, 5], 2, 32
    g = torch.Generator().manual_seed(79)
    N = sum(lengths)
    k = torch.randn(N, HK, D, generator=g).to(torch.bfloat16)
    v = torch.randn(N, HK, D, generator=g).to(torch.bfloat16)
    cu = [0, 3, 4, 9]
    kq, ks, vq, vs = oracle.cache_image_fp8(k, v, cu)
    assert kq.dtype == np.uint8 and kq.shape == (N * HK * D,) and ks.shape == (N * HK,)
    for b, L in enumerate(lengths):
        for hk in range(HK):
            for t in range(L):
                row = cu[b] * HK + hk * L + t
                ck, sk = oracle.quantize_rows_fp8(k[cu[b] + t, hk].view(1, D))
                cv, sv = oracle.quantize_rows_fp8(v[cu[b] + t, hk].view(1, D))
                assert np.array_equal(kq[row * D:(row + 1) * D], ck[0]) and ks[row] == sk[0]
                assert np.array_equal(vq[row * D:(row + 1) * D], cv[0]) and vs[row] == sv[0]


# ---------------------------------------------------------------- paged cache
# Paged KV cache ("大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.2,
# untitled page www.zwxr.cn/news/300951 §3.4: 16-token blocks, not contiguous,
# located through a block table; requests with a common prefix may share
# blocks).  Reading: blocks [num_blocks, HK, 16, D], position j of sequence b in
# block table[b][j // 16], row j % 16.

def _paged_from_slab(slab, bt, num_blocks):
    """Scatter a [B, HK, cap, D] slab into [num_blocks, HK, 16, D] pages."""
    B, HK, cap, D = slab.shape
    pages = torch.zeros((num_blocks, HK, 16, D), dtype=slab.dtype)
    for b in range(B):
        for i in range(cap // 16):
            pages[bt[b][i]] = slab[b, :, 16 * i:16 * (i + 1)]
    return pages


def _slab_from_paged(pages, bt, cap):
    B = len(bt)
    HK, D = pages.shape[1], pages.shape[3]
    slab = np.zeros((B, HK, cap, D), np.uint16)
    for b in range(B):
        for i in range(cap // 16):
            slab[b, :, 16 * i:16 * (i + 1)] = pages[bt[b][i]]
    return slab


def _chunked_case(seed, lengths, prefix, cap, H, HK, D):
    g = torch.Generator().manual_seed(seed)
    N = sum(lengths)
    q = torch.randn(N, H, D, generator=g).to(torch.bfloat16)
    k = torch.randn(N, HK, D, generator=g).to(torch.bfloat16)
    v = torch.randn(N, HK, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(len(lengths), HK, cap, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(len(lengths), HK, cap, D, generator=g).to(torch.bfloat16)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return q, k, v, cu, kc, vc


@pytest.mark.parametrize("H,HK", [(4, 4), (4, 2)])
def test_paged_equals_slab_under_block_permutation(H, HK):
    """Any placement of the blocks gives the slab layout's outputs exactly, and
    the written pages, read back through the table, are the slab image."""
    lengths, prefix, cap, D = [5, 1, 40, 17], [33, 80, 0, 16], 96, 32
    q, k, v, cu, kc, vc = _chunked_case(90 + H + HK, lengths, prefix, cap, H, HK, D)
    B, nbps = len(lengths), cap // 16
    perm = np.random.default_rng(91).permutation(B * nbps + 7)[:B * nbps]
    bt = perm.reshape(B, nbps).astype(np.int32)
    nblocks = B * nbps + 7
    kp = _paged_from_slab(kc, bt, nblocks)
    vp = _paged_from_slab(vc, bt, nblocks)
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, prefix, kc, vc, 0.2)
    out, kpi, vpi = oracle.prefill_chunked_paged(q, k, v, cu, prefix, kp, vp, bt, 0.2)
    assert np.array_equal(out, ref)
    assert np.array_equal(_slab_from_paged(kpi, bt, cap), kimg.reshape(B, HK, cap, D))
    assert np.array_equal(_slab_from_paged(vpi, bt, cap), vimg.reshape(B, HK, cap, D))
    # blocks no sequence maps are untouched
    unused = sorted(set(range(nblocks)) - set(bt.reshape(-1).tolist()))
    assert np.array_equal(kpi[unused], kp[unused].view(torch.int16).numpy().view(np.uint16))


def test_paged_shared_prefix_blocks():
    """Two requests with the same 32-token prefix share its two physical
    blocks; each gets what it would get with a private copy."""
    H, D = 2, 32
    g = torch.Generator().manual_seed(92)
    pk = torch.randn(32, H, D, generator=g).to(torch.bfloat16)
    pv = torch.randn(32, H, D, generator=g).to(torch.bfloat16)
    lengths, prefix = [3, 1], [32, 32]
    q = torch.randn(4, H, D, generator=g).to(torch.bfloat16)
    k = torch.randn(4, H, D, generator=g).to(torch.bfloat16)
    v = torch.randn(4, H, D, generator=g).to(torch.bfloat16)
    cu = [0, 3, 4]
    slab_k = torch.zeros(2, H, 48, D, dtype=torch.bfloat16)
    slab_v = torch.zeros_like(slab_k)
    slab_k[:, :, :32] = pk.transpose(0, 1)
    slab_v[:, :, :32] = pv.transpose(0, 1)
    ref, _, _, _ = oracle.prefill_chunked(q, k, v, cu, prefix, slab_k, slab_v, 0.3)
    bt = np.array([[0, 1, 2], [0, 1, 3]], np.int32)  # blocks 0, 1 shared
    kp = torch.zeros(4, H, 16, D, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    for i in range(2):
        kp[i] = pk[16 * i:16 * (i + 1)].transpose(0, 1)
        vp[i] = pv[16 * i:16 * (i + 1)].transpose(0, 1)
    out, kpi, _ = oracle.prefill_chunked_paged(q, k, v, cu, prefix, kp, vp, bt, 0.3)
    assert np.array_equal(out, ref)
    kb = k.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kpi[2][:, :3], kb[0:3].transpose(1, 0, 2))  # request 0's new tokens
    assert np.array_equal(kpi[3][:, :1], kb[3:4].transpose(1, 0, 2))  # request 1's new token


def test_paged_rejects_bad_block_ids():
    q, k, v, cu, kc, vc = _chunked_case(93, [2], [20], 32, 2, 2, 32)
    kp = _paged_from_slab(kc, np.array([[0, 1]]), 2)
    with pytest.raises(Exception):
        oracle.prefill_chunked_paged(q, k, v, cu, [20], kp, kp, np.array([[0, 2]], np.int32), 0.1)
    with pytest.raises(Exception):
        oracle.prefill_chunked_paged(q, k, v, cu, [20], kp, kp, np.array([[-1, 0]], np.int32), 0.1)
