"""The build's scratch-memory check reads the compiler's resource-usage
remarks; a kernel with a nonzero ScratchSize must be reported."""
from group_quantized_weight_amd import build


def test_scratch_kernels_parsed():
    remarks = "\n".join([
        "a.hip:1:1: remark: Function Name: _Z1fv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 40 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _Z1gv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 48 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._scratch_kernels(remarks) == [("_Z1gv", 48)]
    assert build._scratch_kernels("") == []
