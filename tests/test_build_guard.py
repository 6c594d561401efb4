"""The build refuses kernels that spill registers or use scratch memory
(parsed from the compiler's kernel-resource-usage remarks)."""
import pytest

from decode_attention_paged_amd import build

REMARKS = """\
x.hip:10:1: remark: Function Name: good_kernel [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     AGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     SGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark: Function Name: spilling_kernel [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs Spill: 15 [-Rpass-analysis=kernel-resource-usage]
""".splitlines()


def test_remarks_are_parsed_per_kernel():
    u = build.resource_usage(REMARKS)
    assert u["good_kernel"] == {"VGPRs": 256, "AGPRs": 256, "ScratchSize": 0, "SGPRs Spill": 12,
                                "VGPRs Spill": 0}
    assert u["spilling_kernel"]["ScratchSize"] == 64
    assert u["spilling_kernel"]["VGPRs Spill"] == 15


def test_spills_and_scratch_are_refused():
    u = build.resource_usage(REMARKS)
    with pytest.raises(RuntimeError, match="spilling_kernel"):
        build.check_usage(u)
    build.check_usage({"good_kernel": u["good_kernel"]})   # SGPR spills to VGPR lanes are fine
