"""CPU test of the device code's resource use, from a device-only gfx950
compile (no GPU needed): no kernel spills vector registers or uses scratch
memory, and the step kernel keeps the occupancy its grid sizing assumes
(two 4-wave workgroups per CU for bf16 K/V and for d = 64, one for fp32
K/V at d = 128).  A spill in the step kernel slows every step it runs
without changing a result, so parity tests cannot see it."""

import os
import shutil

import pytest

from shared_prefix_paged_contiguous_amd import build


@pytest.fixture(scope="module")
def usage():
    if not (os.path.exists(build.hipcc()) or shutil.which(build.hipcc())):
        pytest.skip("hipcc not found")
    return build.resource_usage()


def test_every_kernel_is_reported(usage):
    names = list(usage)
    for kernel in ("step_kernel", "append_kernel", "hot_write_kernel", "zero_kernel", "read_kernel"):
        assert any(kernel in n for n in names), kernel
    # T in {bf16, fp32} x D in {64, 128} x RB x partials x two argument capacities
    assert sum("step_kernel" in n for n in names) == 20


def test_no_kernel_spills_or_uses_scratch(usage):
    bad = {n: u for n, u in usage.items() if u.get("VGPRs Spill", 0) or u.get("ScratchSize", 0)}
    assert not bad, bad


def test_step_kernel_occupancy(usage):
    for name, u in usage.items():
        if "step_kernel" not in name:
            continue
        fp32_d128 = "step_kernelIfLi128" in name
        assert u["Occupancy"] == (1 if fp32_d128 else 2), (name, u)
        assert u["LDS Size"] <= (98304 if fp32_d128 else 65536), (name, u)
