"""Register, scratch and occupancy figures of the gfx950 kernels, read from
the compiler's resource-usage remarks on a device-only build of the kernel
source with the library's own flags (no GPU needed).

Every kernel must run without scratch memory (no spilled registers), and the
single-pass kernels with 16 vectors per thread -- which update their state
two vectors at a time -- must keep two waves per SIMD: the 512-thread
workgroup needs it to launch at all, and the 256-thread one to put two
workgroups on a CU. Their register count is pinned to the allocation whose
speed was measured (230 VGPRs): a compiler or source change that moves it
fails here, to be measured again, instead of changing the kernel's speed
silently."""
import os
import re
import shutil
import subprocess

import pytest

from sharded_optimizer_step_amd import _build

PINNED_VGPRS = {("0", "512", "16"): 230, ("0", "256", "16"): 230}


def remarks():
    src = os.path.join(_build.CSRC, "zero_kernels.hip")
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = ["hipcc", *flags, "--cuda-device-only", "-c", "-o", os.devnull, "-I", os.path.join(_build.ROOT, "include"),
           "-I", _build.CSRC, src, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


@pytest.fixture(scope="module")
def usage():
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not found")
    return remarks()


def fused(name):
    """(mode, threads, vectors) of a fused_kernel instantiation, else None."""
    m = re.search(r"fused_kernelILNS_4ModeE(\d)ELi(\d+)ELi(\d+)E", name)
    return m.groups() if m else None


def test_no_kernel_uses_scratch(usage):
    assert len(usage) >= 40
    for name, u in usage.items():
        assert u["ScratchSize"] == "0", (name, u)
        assert u["VGPRs Spill"] == "0", (name, u)


def test_every_fused_kernel_fits_its_workgroup(usage):
    seen = 0
    for name, u in usage.items():
        g = fused(name)
        if g is None:
            continue
        seen += 1
        waves_per_simd = max(1, int(g[1]) // 256)  # a workgroup's waves spread over the CU's four SIMDs
        assert int(u["Occupancy"]) >= waves_per_simd, (g, u)
    assert seen == 25  # the (pass, geometry) pairs the planner can launch


def test_paired_update_kernels_keep_their_measured_allocation(usage):
    for name, u in usage.items():
        g = fused(name)
        if g in PINNED_VGPRS:
            assert int(u["Occupancy"]) >= 2, (g, u)
            assert int(u["VGPRs"]) == PINNED_VGPRS[g], (
                f"{g}: {u['VGPRs']} VGPRs, the measured allocation has {PINNED_VGPRS[g]}: measure the single-pass "
                f"step again before changing the pin")
