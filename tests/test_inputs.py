"""The synthetic workload recipe: generator test vectors and the pages' batching arithmetic."""
import json
import os

import numpy as np
import torch

from prefill_self_attention_amd import inputs as I

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "pages_worked_examples.json")))


def test_splitmix64_published_vectors():
    s = I.SplitMix64(0)
    assert [s.next() for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    s = I.SplitMix64(1234567)
    assert [s.next() for _ in range(3)] == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_decode_contexts_recipe():
    c = I.decode_contexts(4)
    assert len(c) == 64 and sum(c) == 151148 and min(c) == 265 and max(c) == 4040
    assert c[:5] == [1913, 3683, 3555, 2144, 1771]
    assert all(256 <= x <= 4096 for x in c)


def test_longmix_recipe():
    L = I.loguniform_lengths(5)
    assert L == [714, 6988, 273, 118, 206, 687, 29945, 1552, 915, 2760, 1063, 150, 14954, 1078,
                 4133, 32768]
    assert sum(L[:-1]) == 65536 and sum(L) == 98304
    assert all(64 <= x <= 32768 for x in L)


def test_cu_seqlens_from_pages():
    fx = GOLDEN["varlen_metadata"]
    assert I.cu_from_lengths(fx["lengths"]) == fx["cu_seqlens"]
    assert I.cu_from_lengths(fx["lengths"])[-1] == fx["total_tokens"]


def test_padding_waste_arithmetic_from_pages():
    fx = GOLDEN["varlen_metadata"]
    L = fx["lengths"]
    m = max(L)
    waste = [round(100 * (m - n) / m) for n in L]
    assert waste == fx["padding_waste_percent_by_prompt"]
    fx = GOLDEN["padding_batch_10_50_2048"]
    L, m = fx["lengths"], fx["padded_to"]
    token_waste = 1 - sum(L) / (len(L) * m)
    pair_waste = 1 - sum(n * (n + 1) // 2 for n in L) / (len(L) * m * (m + 1) // 2)
    assert round(100 * token_waste, 1) == 65.7
    assert pair_waste * 100 > fx["waste_percent_more_than"]


def test_causal_pair_counts():
    assert 2048 * 2049 // 2 == 2098176
    # 16 chunks of 512 with prefix 512c: sum of pairs = one-shot 8192 prompt
    pairs = sum(512 * 512 * c + 512 * 513 // 2 for c in range(16))
    assert pairs == 8192 * 8193 // 2


def test_values_are_seeded_bf16_normal():
    w = I.workload("single_T64_H4_D32")
    q1, k1, v1 = w.tensors()
    q2, _, _ = w.tensors()
    assert q1.dtype == torch.bfloat16 and tuple(q1.shape) == (64, 4, 32)
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))
    allv = torch.cat([q1, k1, v1]).float()
    assert abs(allv.mean().item()) < 0.05 and abs(allv.std().item() - 1) < 0.05
    assert w.scale == float(np.float32(1 / np.sqrt(32)))
