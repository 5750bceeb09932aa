"""The library build's resource guard (CPU only; hipcc cross-compiles gfx950).

The mainloop kernel is designed for three waves per SIMD (at most 168 VGPRs)
and no scratch memory: its tile-load waits count exactly the tile loads in
flight, and a register spill would add scratch accesses to the same counter.
The build reads the compiler's kernel-resource-usage report and refuses a
library that breaks either condition; these tests run it on the sources as
they are and on a variant made deliberately register-heavy.
"""
import os
import shutil

import pytest

from quantized_exact_attention_amd import build as lib_build

CSRC = lib_build.CSRC


def test_parser_reads_the_compiler_report():
    text = "\n".join([
        "x.hip:1:1: remark: Function Name: _ZN4sage12_GLOBAL__N_115mainloop_kernelENS_12MainloopArgsE "
        "[-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs: 170 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]",
    ])
    res = lib_build.kernel_resources(text)
    (name, r), = res.items()
    assert "mainloop_kernel" in name
    assert r == {"VGPRs": 170, "AGPRs": 0, "ScratchSize": 12, "Occupancy": 2, "VGPRs Spill": 3}
    problems = lib_build.check_resources(res)
    assert len(problems) == 3          # scratch, registers, occupancy


def test_library_sources_meet_the_limits(tmp_path):
    out = str(tmp_path / "libsage_check.so")
    lib_build.build(force=True, out=out)
    assert os.path.exists(out)


def test_register_heavy_mainloop_fails_the_build(tmp_path):
    """The mainloop built for four workgroups per CU: the compiler either
    spills or gives up the occupancy (it keeps all of the loop's registers and
    runs one wave per SIMD); either way the build refuses it instead of
    producing a library."""
    src = tmp_path / "csrc"
    shutil.copytree(CSRC, src)
    path = src / "attn_mainloop.hip"
    text = path.read_text()
    assert "constexpr int kWavesPerSimd = 3;" in text
    path.write_text(text.replace("constexpr int kWavesPerSimd = 3;", "constexpr int kWavesPerSimd = 4;"))
    out = str(tmp_path / "libsage_heavy.so")
    with pytest.raises(RuntimeError, match="kernel resources out of bounds"):
        lib_build.build(force=True, csrc=str(src), out=out)
    assert not os.path.exists(out)
