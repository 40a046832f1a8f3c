"""The kernels' gfx950 assembly has no uncovered matrix-core hazard.

Compiles the forward kernels' sources to assembly with the library's own flags
(device code only, on the CPU), as built for libattn.so and with
``-DATTN_SINGLE_STAGE`` as built for the single-stage debug library, and scans
every kernel instantiation with ``tests/isa_scan.py``. A positive control plants each hazard in a short
assembly listing and checks that the scan reports it.
"""
import os
import subprocess

import pytest

from tests import isa_scan
from tiled_attention_05_amd import build as B

SOURCES = ["attn_fwd_bf16.hip", "fp8.hip"]


def _asm(src, tmp_path, defines=()):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *B.HIP_FLAGS, *defines, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


@pytest.mark.parametrize("defines", [(), ("-DATTN_SINGLE_STAGE",)], ids=["pipelined", "single_stage"])
@pytest.mark.parametrize("src", SOURCES)
def test_no_uncovered_mfma_hazard(src, defines, tmp_path):
    ks = {k: v for k, v in isa_scan.kernels(_asm(src, tmp_path, defines)).items() if "fwd_" in k}
    assert ks, "no forward kernel found in the assembly"
    bad = {k: isa_scan.scan(v) for k, v in ks.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, "\n".join(f"{k}: {h[:3]}" for k, v in bad.items() for h in v)
    n_mfma = sum(sum(1 for line in v if "v_mfma" in line) for v in ks.values())
    assert n_mfma > 0


def test_scan_reports_planted_hazards():
    early_read = ["v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]",
                  "s_nop 3",
                  "v_accvgpr_read_b32 v20, a3"]
    assert [h[0] for h in isa_scan.scan(early_read)] == ["mfma->read"]
    covered = [early_read[0], "s_nop 7", "s_nop 7", "s_nop 7", early_read[2]]
    assert isa_scan.scan(covered) == []
    early_operand = ["v_cvt_pk_bf16_f32 v7, v30, v31",
                     "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]"]
    assert [h[0] for h in isa_scan.scan(early_operand)] == ["write->mfma"]
    spaced = [early_operand[0], "s_nop 1", early_operand[1]]
    assert isa_scan.scan(spaced) == []
    across_branch = [early_read[0], "s_cbranch_vccnz .LBB0_3", early_read[2]]
    assert isa_scan.scan(across_branch) == []   # straight-line scope, by design
