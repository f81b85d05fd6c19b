"""MFMA instructions ignore the EXEC mask, so no MFMA may sit in a region of
the gfx950 code where EXEC has been narrowed for a branch.  A guard that the
compiler lowers to EXEC masking (because it cannot see that the condition is
wave-uniform) would let the MFMA run for the whole wave anyway.

This compiles the kernels to gfx950 assembly (no GPU needed) and checks every
MFMA.
"""
import os
import re
import subprocess

import pytest

from mixture_experts_layer_up_amd import build

SOURCES = [f for f in build.sources() if "expert_gemm" in f]


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [build.HIPCC, *build.COMMON_FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _mfma_under_exec_mask(asm):
    """(kernel, line) of every MFMA issued while EXEC is narrowed."""
    bad, total = [], 0
    kernel, masked = None, False
    for ln in asm.splitlines():
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            kernel, masked = m.group(1), False
            continue
        t = ln.strip()
        if t.startswith("s_and_saveexec") or t.startswith("s_andn2_saveexec"):
            masked = True
        elif re.match(r"s_(or|mov)_b64\s+exec,", t):
            masked = False
        elif t.startswith("v_mfma"):
            total += 1
            if masked:
                bad.append((kernel, t))
        elif t.startswith("s_endpgm"):
            kernel, masked = None, False
    return bad, total


@pytest.mark.parametrize("src", SOURCES, ids=os.path.basename)
def test_no_mfma_under_exec_mask(src, tmp_path):
    bad, total = _mfma_under_exec_mask(_device_asm(src, tmp_path))
    assert total > 0
    assert not bad, f"{len(bad)} of {total} MFMAs sit under an EXEC mask: {bad[:3]}"
