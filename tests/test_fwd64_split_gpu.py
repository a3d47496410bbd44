"""GPU parity for a lone multi-row sequence through the split-KV chunked call
(prefill_attn_chunked_splitkv with one sequence and max_seqlen > 1, head_dim
128, scale >= 0): the call appends the chunk's K/V rows to the cache, runs the
split-KV items on the 64-row kernel with every key read from the cache, and
merges the segments.  The result is chunked attention
("大模型 Prompt Prefill 阶段的高效 Batching 与算子排布" §3: a prompt prefilled
chunk by chunk over its cached prefix), so the oracle is
oracle.prefill_chunked: outputs to the parity bar of tests/gpu_util.py, cache
bytes bit for bit, nothing written past the workspace.  The prefixes cover
the diagonal at every offset within a 64-key tile (0, 1, 40, 63), items with
one and with several segments, grouped K/V heads and an odd head count."""
import pytest
import torch

from tests.test_splitkv_gpu import check_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefill_self_attention_amd as P
    P.load()
    yield


CASES = [
    # length, prefix, capacity, H, HK
    (512, 7680, 8192, 32, 32),   # the chunked workload's last chunk: four segments per block
    (512, 0, 8192, 8, 8),        # its first chunk, no prefix
    (300, 1000, 2048, 8, 8),     # prefix 1000 (diagonal 40 keys into a tile), ragged rows
    (1000, 63, 2048, 4, 2),      # prefix 63, grouped heads
    (129, 64, 512, 2, 2),        # two blocks, the second with one row
    (700, 1, 4096, 6, 3),        # prefix 1, six heads over three K/V heads
    (200, 500, 1024, 3, 3),      # odd head count: a work-group's two units from different items
    (100, 60000, 70000, 2, 2),   # long prefix: 36-tile segments
]


@pytest.mark.parametrize("n,pre,cap,H,HK", CASES)
def test_fwd64_split_lone_chunk(n, pre, cap, H, HK):
    check_case([n], [pre], cap, H, HK, 128, 1200 + n + pre % 97, "fwd64 split len=%d prefix=%d" % (n, pre))


def test_fwd64_split_decode_row_as_item():
    # one row, max_seqlen above 1: the row runs as a one-row block item
    check_case([1], [777], 1024, 4, 4, 128, 1290, "fwd64 split one row", max_seqlen=4)


@pytest.mark.parametrize("scale", [0.0, 2.0])
def test_fwd64_split_scales(scale):
    check_case([260], [900], 2048, 4, 4, 128, 1295, "fwd64 split scale", scale=scale)


@pytest.mark.parametrize("i", range(12))
def test_fwd64_split_random(i):
    """Seeded random lone chunks: lengths 2..700, prefixes 0..3000 (any offset
    within a tile), grouped and odd head counts, three scales, capacity with
    slack past the chunk."""
    import numpy as np
    from prefill_self_attention_amd import inputs as I
    rng = np.random.default_rng(1300 + i)
    H, HK = [(2, 1), (4, 2), (6, 3), (8, 8), (3, 3), (4, 4)][int(rng.integers(0, 6))]
    n = int(rng.integers(2, 701))
    pre = int(rng.integers(0, 3001))
    cap = pre + n + int(rng.integers(0, 300))
    scale = float([I.default_scale(128), 0.0, 0.7][int(rng.integers(0, 3))])
    check_case([n], [pre], cap, H, HK, 128, 1400 + i, "fwd64 split random %d: len=%d prefix=%d" % (i, n, pre),
               scale=scale)
