"""Host logic of the build's kernel-resource report (CPU only): the
compiler's kernel-resource-usage remarks are parsed into one record per
kernel, and a kernel that uses scratch memory or spills vector registers
makes the build fail."""
import os
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "block_scaled_precision_quant_amd"))
import _build  # noqa: E402

REMARKS = """\
gemm.hip:66:1: remark: Function Name: _ZN2mx11gemm_kernelILi1ELi1ELi1ELi4EEEvNS_8GemmArgsE [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     TotalSGPRs: 94 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     VGPRs: 76 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     Occupancy [waves/SIMD]: 6 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     VGPRs Spill: {vspill} [-Rpass-analysis=kernel-resource-usage]
gemm.hip:66:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


@pytest.fixture
def report_dir(tmp_path, monkeypatch):
    monkeypatch.setattr(_build, "BUILD", str(tmp_path))
    monkeypatch.setattr(_build, "REPORT", str(tmp_path / "kernel_resources.txt"))
    return tmp_path


def test_remarks_parse_into_records(report_dir):
    ks = _build.parse_resources(REMARKS.format(scratch=0, vspill=0), "gemm.hip")
    assert len(ks) == 1
    k = ks[0]
    assert (k["sgpr"], k["vgpr"], k["agpr"], k["scratch"], k["occupancy"]) == (94, 76, 0, 0, 6)
    assert (k["sgpr_spill"], k["vgpr_spill"], k["lds"], k["dynamic_stack"]) == (0, 0, 0, "False")
    _build.write_report(ks)
    text = (report_dir / "kernel_resources.txt").read_text()
    assert "mx::gemm_kernel<1, 1, 1, 4>(mx::GemmArgs)" in text  # demangled


@pytest.mark.parametrize("scratch,vspill", [(16, 0), (0, 4)])
def test_scratch_or_vector_spill_fails_the_build(report_dir, scratch, vspill):
    ks = _build.parse_resources(REMARKS.format(scratch=scratch, vspill=vspill), "gemm.hip")
    with pytest.raises(RuntimeError, match="scratch memory or spilling vector registers"):
        _build.write_report(ks)


def test_built_library_report_is_clean():
    """The report of the last build lists every kernel of the library with no
    scratch use (written by build(); skipped when nothing was built here)."""
    if not os.path.exists(_build.REPORT):
        pytest.skip("no build report in this tree")
    lines = [l for l in open(_build.REPORT) if not l.startswith("#")]
    assert len(lines) >= 120
    for l in lines:
        cols = [c.strip() for c in l.split("|")]
        assert cols[3] == "0", l  # scratch bytes per lane
        assert cols[4].split()[1] == "0", l  # vector-register spills
