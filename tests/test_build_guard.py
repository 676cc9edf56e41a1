"""The build rejects a direct-to-LDS GEMM kernel that touches scratch memory.

That kernel waits on hand-counted vector-memory operations; a compiler spill
(a scratch load or store) between its DMA instructions would shift the counts,
so build.py parses hipcc's resource-usage remarks and refuses such a build.
"""
import pytest

from moe_expert_dispatch_amd import build as b

_DMA = "_ZN3moe12_GLOBAL__N_123grouped_gemm_dma_kernelILi0ELb0ELb0EEEvPK"
_REG = "_ZN3moe12_GLOBAL__N_124grouped_gemm_bf16_kernelILi0EEEvPK"


def _remarks(name, scratch, vspill):
    tag = "[-Rpass-analysis=kernel-resource-usage]"
    return "\n".join([
        f"x.hip:1:1: remark: Function Name: {name} {tag}",
        f"x.hip:1:1: remark:     VGPRs: 200 {tag}",
        f"x.hip:1:1: remark:     ScratchSize [bytes/lane]: {scratch} {tag}",
        f"x.hip:1:1: remark:     VGPRs Spill: {vspill} {tag}",
    ])


def test_clean_dma_kernel_passes():
    b._check_no_scratch("gemm_mfma.hip", _remarks(_DMA, 0, 0))


@pytest.mark.parametrize("scratch,vspill", [(4, 0), (0, 3), (16, 4)])
def test_dma_kernel_with_scratch_is_rejected(scratch, vspill):
    with pytest.raises(RuntimeError, match="grouped_gemm_dma_kernel"):
        b._check_no_scratch("gemm_mfma.hip", _remarks(_DMA, scratch, vspill))


def test_other_kernels_may_spill():
    # compiler-managed waits: a spill costs time, not correctness
    b._check_no_scratch("gemm_mfma.hip", _remarks(_REG, 12, 0) + "\n" + _remarks(_DMA, 0, 0))
