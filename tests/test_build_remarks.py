"""build.py reports kernels that use scratch memory, from hipcc's
kernel-resource-usage remarks (CPU only: parses sample remark text)."""
from prefill_self_attention_amd import build

SAMPLE = """\
x.hip:10:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
y.hip:20:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
y.hip:20:1: remark:     ScratchSize [bytes/lane]: 36 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_reports_only_nonzero_scratch():
    assert build.scratch_kernels(SAMPLE) == [("kern_b", 36)]


def test_scratch_kernels_empty_text():
    assert build.scratch_kernels("") == []
