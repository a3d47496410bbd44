"""Concurrent calls: the header states that calls are re-entrant and run on
the caller's stream.  Four host threads, each with its own stream, buffers
and split-KV workspace, call every entry point repeatedly at the same time;
every result must equal, bit for bit, the one the same call gave alone on the
default stream (same inputs, same work split, so the same arithmetic)."""
import threading

import numpy as np
import pytest
import torch

from prefill_self_attention_amd import inputs as I
from tests.gpu_util import bits, say

pytestmark = pytest.mark.gpu

THREADS = 4
REPEATS = 5


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


def make_problem(seed):
    """A varlen batch, a chunked batch (a chunk, decode rows) with its slab
    cache, all on the device."""
    H, HK, D = 8, 2, 128
    g = I.generator(seed)
    lengths = [300, 1, 77, 1, 129]
    cu = I.cu_from_lengths(lengths)
    N = cu[-1]
    q = I.randn_bf16(g, (N, H, D)).cuda()
    k = I.randn_bf16(g, (N, HK, D)).cuda()
    v = I.randn_bf16(g, (N, HK, D)).cuda()
    prefix = [700, 1500, 64, 3000, 0]
    cap = 16 * ((max(p + n for p, n in zip(prefix, lengths)) + 15) // 16)
    kc0 = I.randn_bf16(g, (len(lengths), HK, cap, D)).cuda()
    vc0 = I.randn_bf16(g, (len(lengths), HK, cap, D)).cuda()
    return dict(H=H, HK=HK, D=D, N=N, cap=cap, q=q, k=k, v=v,
                cu=torch.tensor(cu, dtype=torch.int32, device="cuda"),
                pre=torch.tensor(prefix, dtype=torch.int32, device="cuda"),
                kc0=kc0, vc0=vc0, max_len=max(lengths), B=len(lengths))


def run_all(pb, ws):
    """Every entry point once on the current stream; returns the device results."""
    m = P()
    res = {}
    N, HK, D = pb["N"], pb["HK"], pb["D"]
    out = torch.empty_like(pb["q"])
    kc = torch.empty(N * HK * D, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    m.prefill_attn_varlen(pb["q"], pb["k"], pb["v"], pb["cu"], kc, vc, out, max_seqlen=pb["max_len"])
    res["varlen"] = (out, kc, vc)
    out = torch.empty_like(pb["q"])
    kq = torch.empty(N * HK * D, dtype=torch.int8, device="cuda")
    vq = torch.empty_like(kq)
    ks = torch.empty(N * HK, dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    m.prefill_attn_varlen_int8(pb["q"], pb["k"], pb["v"], pb["cu"], kq, vq, ks, vs, out, max_seqlen=pb["max_len"])
    res["int8"] = (out, kq, vq, ks, vs)
    out = torch.empty_like(pb["q"])
    kf = torch.empty(N * HK * D, dtype=torch.uint8, device="cuda")
    vf = torch.empty_like(kf)
    ks = torch.empty(N * HK, dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    m.prefill_attn_varlen_fp8(pb["q"], pb["k"], pb["v"], pb["cu"], kf, vf, ks, vs, out, max_seqlen=pb["max_len"])
    res["fp8"] = (out, kf, vf, ks, vs)
    out = torch.empty_like(pb["q"])
    kc, vc = pb["kc0"].clone(), pb["vc0"].clone()
    m.prefill_attn_chunked(pb["q"], pb["k"], pb["v"], pb["cu"], kc, vc, out, pb["pre"], max_seqlen=pb["max_len"])
    res["chunked"] = (out, kc, vc)
    out = torch.empty_like(pb["q"])
    kc, vc = pb["kc0"].clone(), pb["vc0"].clone()
    m.prefill_attn_chunked_splitkv(pb["q"], pb["k"], pb["v"], pb["cu"], kc, vc, out, pb["pre"],
                                   max_seqlen=pb["max_len"], workspace=ws)
    res["splitkv"] = (out, kc, vc)
    # one query head per K/V head: the decode rows run inside the attention
    # launch, whose work-groups take items and units from shared counters
    q1 = pb["q"][:, :HK].contiguous()
    out = torch.empty_like(q1)
    kc, vc = pb["kc0"].clone(), pb["vc0"].clone()
    m.prefill_attn_chunked_splitkv(q1, pb["k"], pb["v"], pb["cu"], kc, vc, out, pb["pre"],
                                   max_seqlen=pb["max_len"], workspace=ws)
    res["splitkv_mixed"] = (out, kc, vc)
    return res


def to_host(res):
    return {name: [bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy().copy() for t in ts]
            for name, ts in res.items()}


def test_concurrent_threads_own_streams():
    pb = make_problem(1200)
    wsz = P().splitkv_workspace_size(pb["B"], pb["N"], pb["H"], pb["D"], pb["cap"])
    say("case concurrency: reference calls")
    ws0 = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    ref = to_host(run_all(pb, ws0))
    torch.cuda.synchronize()

    errors = []
    results = [None] * THREADS

    def worker(t):
        try:
            s = torch.cuda.Stream()
            ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
            got = []
            with torch.cuda.stream(s):
                for _ in range(REPEATS):
                    got.append(run_all(pb, ws))
            s.synchronize()
            results[t] = [to_host(r) for r in got]
        except Exception as e:  # reported on the main thread
            errors.append(repr(e))

    say("case concurrency: %d threads x %d rounds" % (THREADS, REPEATS))
    ths = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(THREADS):
        for r, got in enumerate(results[t]):
            for name, arrays in ref.items():
                for i, a in enumerate(arrays):
                    np.testing.assert_array_equal(got[name][i], a, err_msg="thread %d round %d %s[%d]" % (t, r, name, i))
