"""The build refuses kernels with register spills (their inline-asm products
and DMA rely on no spill code in the loops)."""
from io_aware_exact_flash_amd import build


def test_spill_remarks_are_detected():
    txt = (
        "a.hip:1:1: remark: Function Name: k1 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:2:1: remark: Function Name: k2 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:2:1: remark:     VGPRs Spill: 21 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:2:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
    )
    bad = build._spills(txt)
    assert len(bad) == 1 and bad[0].startswith("k2")


def test_no_spill_remarks_pass():
    assert build._spills("x.hip:1:1: remark: Function Name: k [-Rpass]\n"
                         "x.hip:1:1: remark: VGPRs Spill: 0 [-Rpass]\n") == []
