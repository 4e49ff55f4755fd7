"""The build's register-spill check (host logic only): the compiler's
kernel-resource-usage remarks are parsed per kernel, and a kernel outside the
listed ceilings fails the build on any spill or scratch use."""
from bitwise_deterministic_exact_pass1_amd import build as B

REMARKS = """\
x.hip:10:1: remark: Function Name: _ZN3det10k_finalizeEv [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     TotalSGPRs: 78 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark: Function Name: _ZN3det9k_qk_mfmaILi2EEEvNS_6QkArgsE [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     SGPRs Spill: 20 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parses_every_kernel():
    res = B.kernel_resources(REMARKS)
    assert res == {"_ZN3det10k_finalizeEv": (0, 0, 0), "_ZN3det9k_qk_mfmaILi2EEEvNS_6QkArgsE": (20, 0, 0)}
    assert B.spill_violations(res) == []


def test_unlisted_kernel_with_any_spill_or_scratch_fails():
    for got in [(1, 0, 0), (0, 1, 0), (0, 0, 4)]:
        bad = B.spill_violations({"_ZN3det10k_finalizeEv": got})
        assert len(bad) == 1 and "k_finalize" in bad[0]


def test_listed_kernel_over_its_ceiling_fails():
    lim = next(c for pat, c in B.SPILL_CEILINGS if "k_qk_mfma" in pat)
    assert B.spill_violations({"_ZN3det9k_qk_mfmaILi2EEEvNS_6QkArgsE": lim}) == []
    over = (lim[0] + 1, lim[1], lim[2])
    assert len(B.spill_violations({"_ZN3det9k_qk_mfmaILi2EEEvNS_6QkArgsE": over})) == 1
