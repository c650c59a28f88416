"""Host checks of the build script (no GPU)."""
import re

from sparse_attention_backward_amd import build


def test_scratch_guard_parses_the_resource_remarks():
    remarks = "\n".join([
        "a.hip:1:1: remark: Function Name: kernel_a [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 200 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark: Function Name: kernel_b [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.scratch_users(remarks) == ["kernel_b"]
    assert build.scratch_users("") == []


def test_hand_counted_waits_are_guarded():
    """Every unit whose kernels count their own global->LDS transfers in vmcnt (inline asm
    global_load_lds followed by waits other than vmcnt(0)) is built with the scratch guard."""
    import os
    names = {u[0]: u[1] for u in build.UNITS}
    for name, src in names.items():
        text = open(os.path.join(build.CSRC, src)).read()
        counted = "global_load_lds" in text and re.search(r"wait_vm\w*\s*\(|wait_vmcnt<", text)
        if counted:
            assert name in build.NO_SCRATCH, name
