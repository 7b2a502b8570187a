"""The build's spill guard: the device compiler's kernel-resource-usage
remarks are parsed per kernel, and any scratch use outside the allow-list
fails the build (a spilled matrix-core operand has been seen to be
reloaded only in part, with wrong results and no error)."""
from bwd_causal_flash_amd import build as b

ALLOWED = next(iter(b.SPILL_ALLOWED))

SAMPLE = f"""\
x.hip:48:1: remark: Function Name: _ZN3cpa4fooEv [-Rpass-analysis=kernel-resource-usage]
x.hip:48:1: remark:     VGPRs: 31 [-Rpass-analysis=kernel-resource-usage]
x.hip:48:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark: Function Name: _ZN3cpa4barEv [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:70:1: remark: Function Name: {ALLOWED} [-Rpass-analysis=kernel-resource-usage]
x.hip:70:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_remarks_parsed_per_kernel():
    got = b.scratch_by_kernel(SAMPLE)
    assert got == {"_ZN3cpa4fooEv": 0, "_ZN3cpa4barEv": 12, ALLOWED: 16}


def test_spills_outside_the_allow_list_are_refused():
    bad = b.spill_check(b.scratch_by_kernel(SAMPLE))
    assert bad == ["_ZN3cpa4barEv: 12 bytes/lane"]
    assert b.spill_check({ALLOWED: b.SPILL_ALLOWED[ALLOWED]}) == []
    assert b.spill_check({ALLOWED: b.SPILL_ALLOWED[ALLOWED] + 4}) != []
    assert b.spill_check({"_ZN3cpa4fooEv": 0}) == []


def test_build_asks_for_the_report():
    assert "-Rpass-analysis=kernel-resource-usage" in b.REMARKS
