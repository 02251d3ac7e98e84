"""Instruction-level guard of the epilogue's rounding order (no GPU needed).

The W8A8 epilogue computes fp32(A) * fp32(s_X s_W) rounded to fp32, then to
fp16 (the oracle's order).  The compiler may fold an fp32 product and its
conversion to fp16 into one mixed-precision FMA (v_fma_mixlo_f16 /
v_fma_mixhi_f16), which rounds the exact product once -- a different fp16
value in rare cases -- and it did so in the band kernel until the product was
pinned with as_fp32.  This test compiles the sources that hold the scale
epilogues (and the LoRA weight scaling) for gfx950 and checks that no such
instruction appears.  Mixed FMAs with an fp32 result (v_fma_mix_f32, whose
fp16 inputs widen exactly) are allowed.
"""

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rotation_quantized_int8_amd", "csrc")
sys.path.insert(0, os.path.join(ROOT, "rotation_quantized_int8_amd"))

SOURCES = ["band.hip", "narrow.hip", "gemm_dma.hip", "gemm.hip", "skinny.hip", "lora.hip", "prologue.hip"]
FP16_RESULT_MIX = re.compile(r"\bv_(fma|mad)_mix(lo|hi)_f16\b")


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_single_rounding_fp16_fma_in_epilogues(src, tmp_path):
    import build   # the package's build flags
    out = tmp_path / (src + ".s")
    cmd = [_hipcc(), *build.HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    asm = out.read_text()
    assert "v_mfma" in asm or "v_" in asm          # device code was produced
    hits = [ln.strip() for ln in asm.splitlines() if FP16_RESULT_MIX.search(ln)]
    assert not hits, f"{src}: {len(hits)} mixed-precision FMAs with an fp16 result, e.g. {hits[:3]}"
