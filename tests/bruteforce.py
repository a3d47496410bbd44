"""Brute-force attention in numpy float64 with a materialised causal mask.

An independent second route to the oracle's result, used only on tiny inputs:
the whole score matrix of one (sequence, head) is formed with a matrix product,
entries above the (bottom-right aligned) diagonal are set to -inf, and the
softmax is taken row by row before multiplying by V.  [P4 §2.2: attention is
softmax(Q K^T / sqrt(d_k)) V with each row normalised over the whole row;
P5 §1.1 / §3.3: lower-triangular causal mask.]
[P4] "大语言模型推理核心：Prefill与Decode原理及工程优化"; [P5] page at
www.zwxr.cn/news/300951.
"""
import numpy as np


def bf16_to_f64(bits):
    bits = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def attention_one(q, k, v, scale, prefix=0):
    """q [n, D], k/v [prefix + n, D] float64 -> (out [n, D], probs [n, prefix + n])."""
    n = q.shape[0]
    nk = k.shape[0]
    s = (q @ k.T) * float(scale)
    i = np.arange(n)[:, None]
    j = np.arange(nk)[None, :]
    s = np.where(j <= prefix + i, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v, p


def varlen(q, k, v, cu, scale):
    """q/k/v bf16 bits [N, H, D]; returns float64 [N, H, D]."""
    q, k, v = bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v)
    out = np.zeros_like(q)
    H = q.shape[1]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        for h in range(H):
            out[s:e, h], _ = attention_one(q[s:e, h], k[s:e, h], v[s:e, h], scale)
    return out
