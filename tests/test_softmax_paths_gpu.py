"""GPU parity for the rare paths of the head_dim-128 kernel's online softmax
(the 64-row kernel, varlen and the split-KV items of a lone chunk), on inputs
built to reach them.  The common path computes a tile's weights against the
running max without the tile's own max and checks each lane's sum of them;
the exact path (the row max, the move of the running max, O and l rescaled)
runs when that sum passes its bound.  Online softmax with rescaling is the
blockwise form of one softmax ("Prefill不是热身：大模型推理的真正瓶颈与优化核心" §4:
attention computed tile by tile), so the result must still be the oracle's
softmax(scale · q kᵀ) V to the parity bar of tests/gpu_util.py.

Scores are steered through head-dim column 0: q[:, :, 0] = a and
k[j, :, 0] = f(j) add a·f(j) to the score of key j for every query, on top
of N(0, 1) noise in the other 127 columns."""
import numpy as np
import pytest
import torch

import oracle
from prefill_self_attention_amd import inputs as I
from tests.gpu_util import SENTINEL, assert_close, bits, guards_intact, say
from tests.test_parity_gpu import run_varlen
from tests.test_splitkv_gpu import run_split, sentinel_cache, workspace_for

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefill_self_attention_amd as P
    P.load()
    yield


def steered(lengths, H, seed, a, f):
    """q, k, v ~ N(0, 1) bf16 with q[:, :, 0] = a and k[j, :, 0] = f(position
    of j in its sequence)."""
    g = I.generator(seed)
    cu = I.cu_from_lengths(lengths)
    N = cu[-1]
    q = I.randn_bf16(g, (N, H, D))
    k = I.randn_bf16(g, (N, H, D))
    v = I.randn_bf16(g, (N, H, D))
    q[:, :, 0] = a
    for b, n in enumerate(lengths):
        pos = torch.arange(n, dtype=torch.float32)
        k[cu[b]:cu[b + 1], :, 0] = f(pos)[:, None].to(torch.bfloat16)
    return cu, q, k, v


def check_varlen_steered(lengths, H, seed, a, f, what):
    cu, q, k, v = steered(lengths, H, seed, a, f)
    scale = I.default_scale(D)
    say("case %s lengths=%s H=%d" % (what, lengths, H))
    out, kc, vc, wholes = run_varlen(q, k, v, cu, scale)
    n = cu[-1] * H * D
    sent = np.full(n, SENTINEL, np.uint16)
    ref, kimg, vimg, _ = oracle.prefill_varlen(q, k, v, cu, scale, k_cache=sent, v_cache=sent)
    assert_close(out, ref, what)
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)
    assert all(guards_intact(x) for x in wholes)


def test_scores_growing_every_tile():
    # key j scores 4 j above the noise: about 33 more (exp2 domain) per
    # 64-key tile, so every tile after a row's first passes the running max
    # by far more than the common path allows
    check_varlen_steered([1024, 300, 65], 2, 2001, 4.0, lambda p: 1.0 * p, "growing scores")


def test_score_jump_overflows_common_path():
    # keys from position 500 on score 2400 above the rest (about 306 in the
    # exp2 domain): the common path's weights overflow to inf there
    check_varlen_steered([700, 129], 2, 2002, 4.0, lambda p: torch.where(p >= 500, 600.0, 0.0), "score jump")


def test_score_drop_after_first_tile():
    # the first 64 keys score 2400 above the later ones: the later keys'
    # weights underflow to zero against the running max
    check_varlen_steered([600], 2, 2003, 4.0, lambda p: torch.where(p < 64, 600.0, 0.0), "score drop")


def test_scores_growing_split_lone_chunk():
    # the same growth on the split-KV items of a lone chunk (no prefix: every
    # key is one of the chunk's rows, read back from the cache)
    lengths, H, cap = [900], 4, 1024
    cu, q, k, v = steered(lengths, H, 2004, 4.0, lambda p: 1.0 * p)
    g = I.generator(2005)
    kc0 = sentinel_cache(g, 1, H, cap, D, [0])
    vc0 = sentinel_cache(g, 1, H, cap, D, [0])
    scale = I.default_scale(D)
    say("case growing scores, split lone chunk len=%d H=%d" % (lengths[0], H))
    whole, need = workspace_for(1, cu[-1], H, D, cap)
    kc, vc = kc0.cuda(), vc0.cuda()
    out = run_split(q, k, v, cu, [0], kc, vc, scale, ws=whole[:need])
    ref, kimg, vimg, _ = oracle.prefill_chunked(q, k, v, cu, [0], kc0, vc0, scale)
    assert_close(out, ref, "growing scores, split")
    np.testing.assert_array_equal(bits(kc), kimg)
    np.testing.assert_array_equal(bits(vc), vimg)
