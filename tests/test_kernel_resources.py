"""Register and scratch use of the attention kernels, from the compiler's
resource report for gfx950 (no GPU needed): every attention instance runs at
2 waves per SIMD (2 workgroups of 4 waves per CU) and no kernel of attn.hip
spills to scratch memory, whose per-lane traffic would sit on the step
loops' path."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_attention_19_amd import build_lib as bl  # noqa: E402

SRC = os.path.join(bl.CSRC, "attn.hip")


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(bl.HIPCC):
        pytest.skip("hipcc not available")
    cmd = [bl.HIPCC, *bl.COMMON, f"-I{bl.CSRC}", *bl.DEVICE_FLAGS["attn.hip"], "--cuda-device-only",
           "-S", SRC, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
        if cur and m:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_every_kernel_reported(report):
    names = " ".join(report)
    for k in ("attn_kernelILi128ELb0ELb0", "attn_kernelILi128ELb1ELb0", "attn_kernelILi128ELb0ELb1",
              "attn_kernelILi64ELb0ELb0", "attn_kernelILi64ELb1ELb0", "attn_kernelILi64ELb0ELb1",
              "plan_kernelILb0", "plan_kernelILb1", "combine_kernelILi128", "combine_kernelILi64"):
        assert k in names, k


def test_no_scratch(report):
    for name, r in report.items():
        assert r.get("ScratchSize", 0) == 0, (name, r)
        assert r.get("VGPRs Spill", 0) == 0, (name, r)


def test_attention_occupancy(report):
    for name, r in report.items():
        if "attn_kernel" in name:
            assert r.get("Occupancy", 0) >= 2, (name, r)
            assert r.get("VGPRs", 999) <= 256, (name, r)
