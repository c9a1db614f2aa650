"""The direct global -> LDS loads (dma16, dma16_at, dma16_once) set M0 in inline assembly
that declares M0 clobbered instead of saving and restoring it. That is sound only while the
compiler itself never writes M0 in the kernels that use them (it reserves M0 and would not
restore a value of its own kept across the statement). This compiles each such source to
gfx950 assembly with the library's own flags and checks that every instruction naming M0
lies inside an inline-assembly region."""
import os
import re
import subprocess

import pytest

from exact_tiled_attention_08_amd import build as B

M0 = re.compile(r"\bm0\b")


def _asm(src: str, tmp_path) -> str:
    out = os.path.join(tmp_path, os.path.basename(src) + ".s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    assert "reserved registers" not in res.stderr, "the M0 clobber warning is not silenced"
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_bwd.hip"])
def test_compiler_never_writes_m0(src, tmp_path):
    text = _asm(src, str(tmp_path))
    inside = False
    in_asm = outside = 0
    for line in text.splitlines():
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
            continue
        if s.startswith(";;#ASMEND"):
            inside = False
            continue
        code = s.split(";", 1)[0]
        if not M0.search(code):
            continue
        if inside:
            in_asm += 1
        else:
            outside += 1
            pytest.fail(f"{src}: the compiler uses M0 outside inline assembly: {s}")
    assert in_asm > 0 and outside == 0
