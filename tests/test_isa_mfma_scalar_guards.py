"""Properties of the gfx950 assembly that the kernels rely on (no GPU needed).

1. MFMA instructions ignore the EXEC mask, so no MFMA may sit in a region of
   the code where EXEC has been narrowed for a branch.  A guard that the
   compiler lowers to EXEC masking (because it cannot see that the condition
   is wave-uniform) would let the MFMA run for the whole wave anyway.  Every
   MFMA is checked.
2. The direct global->LDS loads are inline assembly that set M0 (the LDS
   address) and issue the load in one statement.  M0 is a register the
   compiler reserves: it is not told that the statement overwrites it, so any
   instruction of its own that reads or writes M0 could see a clobbered
   value.  In the kernels that use those loads, M0 may appear only in the
   statement's own `s_mov_b32 m0` directly followed by its
   `global_load_lds_dwordx4`, and no instruction that reads M0 implicitly
   (relative moves, messages, GWS, LDS parameter loads) may appear at all.
"""
import os
import re
import subprocess

import pytest

from mixture_experts_layer_up_amd import build

# every source with MFMA code (the permute launch also runs the gate_up shrink)
SOURCES = [f for f in build.sources()
           if "expert_gemm" in f or "lora_shrink" in f or "permute" in f]
# every source that includes the direct-load header
DMA_SOURCES = [f for f in build.sources() if '#include "lds_dma.h"' in open(f).read()]


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [build.HIPCC, *build.COMMON_FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


_LABEL = re.compile(r"^(\.LBB\S+|_Z\S+):")
_BRANCH = re.compile(r"^s_(cbranch_\w+|branch)\s+(\S+)")


def _exec_effect(t):
    """New 'EXEC narrowed' state after instruction t, or None if unchanged."""
    if re.match(r"s_(and|andn2|or|xor)_saveexec_b64", t):
        return True
    if re.match(r"s_(xor|andn2|and)_b64\s+exec,", t):
        return True
    if re.match(r"s_(or|mov)_b64\s+exec,", t):
        return False
    return None


def _mfma_under_exec_mask(asm):
    """(kernel, line) of every MFMA that can be reached while EXEC is narrowed.

    The compiler places masked regions out of line and jumps back, so the
    check follows the control flow: the kernel is cut into basic blocks, and
    'EXEC narrowed' is propagated along every edge (a saveexec or an exec
    and/xor/andn2 narrows it, an exec or/mov restores it; the taken edge of
    s_cbranch_execz exists only while it is narrowed) until nothing changes.
    """
    bad, total = [], 0
    kernels, cur = [], None
    for ln in asm.splitlines():
        t = ln.split(";")[0].strip()
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            cur = (m.group(1), [])
            kernels.append(cur)
            continue
        if cur is None:
            continue
        if t.startswith("s_endpgm"):
            cur[1].append(t)
            cur = None
            continue
        if t:
            cur[1].append(t)
    for name, lines in kernels:
        blocks, labels = [[]], {}
        for t in lines:
            lab = re.match(r"^(\.LBB\S+):", t)
            if lab:
                if blocks[-1]:
                    blocks.append([])
                labels[lab.group(1)] = len(blocks) - 1
                continue
            blocks[-1].append(t)
            if _BRANCH.match(t) or t.startswith("s_endpgm"):
                blocks.append([])
        entry = [False] * len(blocks)
        seen = [False] * len(blocks)
        seen[0] = True
        work = [0]
        while work:
            b = work.pop()
            state = entry[b]
            succ = []
            falls = True
            for t in blocks[b]:
                eff = _exec_effect(t)
                if eff is not None:
                    state = eff
                br = _BRANCH.match(t)
                if br:
                    kind, target = br.groups()
                    # s_cbranch_execz is taken only when EXEC is empty, which
                    # cannot happen while it is whole: that edge exists only
                    # inside a narrowed region
                    if target in labels and (kind != "cbranch_execz" or state):
                        succ.append((labels[target], state))
                    if kind == "branch":
                        falls = False
                if t.startswith("s_endpgm"):
                    falls = False
            if falls and b + 1 < len(blocks):
                succ.append((b + 1, state))
            for nb, st in succ:
                if not seen[nb] or (st and not entry[nb]):
                    seen[nb] = True
                    entry[nb] = entry[nb] or st
                    work.append(nb)
        for b, blk in enumerate(blocks):
            state = entry[b]
            for t in blk:
                eff = _exec_effect(t)
                if eff is not None:
                    state = eff
                if t.startswith("v_mfma"):
                    total += 1
                    if state and seen[b]:
                        bad.append((name, t))
    return bad, total


@pytest.mark.parametrize("src", SOURCES, ids=os.path.basename)
def test_no_mfma_under_exec_mask(src, tmp_path):
    bad, total = _mfma_under_exec_mask(_device_asm(src, tmp_path))
    assert total > 0
    assert not bad, f"{len(bad)} of {total} MFMAs sit under an EXEC mask: {bad[:3]}"


# instructions that read M0 without naming it
_IMPLICIT_M0 = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_ordered|s_ttracedata|"
                          r"ds_param|v_interp|s_cbranch_g_fork)")


def _m0_violations(asm):
    lines = [ln.split(";")[0].strip() for ln in asm.splitlines()]
    lines = [t for t in lines if t and not t.startswith(".")]
    bad, pairs = [], 0
    i = 0
    while i < len(lines):
        t = lines[i]
        if re.match(r"^s_mov_b32\s+m0,", t):
            nxt = lines[i + 1] if i + 1 < len(lines) else ""
            if nxt.startswith("global_load_lds_dwordx4"):
                pairs += 1
                i += 2
                continue
            bad.append(t)
        elif re.search(r"\bm0\b", t) or _IMPLICIT_M0.match(t):
            bad.append(t)
        i += 1
    return bad, pairs


@pytest.mark.parametrize("src", DMA_SOURCES, ids=os.path.basename)
def test_m0_only_in_direct_load_statements(src, tmp_path):
    bad, pairs = _m0_violations(_device_asm(src, tmp_path))
    assert pairs > 0
    assert not bad, f"M0 used outside the direct-load statements: {bad[:5]}"


def test_m0_checker_flags_other_uses():
    """The checker itself: a compiler-style M0 write, an implicit reader, and
    an M0 write not followed by the direct load are all flagged."""
    ok = "s_mov_b32 m0, s4\nglobal_load_lds_dwordx4 v[2:3], off\n"
    assert _m0_violations(ok) == ([], 1)
    assert _m0_violations(ok + "s_mov_b32 m0, -1\nds_read_b32 v1, v2\n")[0]
    assert _m0_violations(ok + "v_movrels_b32 v0, v1\n")[0]
    assert _m0_violations(ok + "v_readlane_b32 s0, v1, m0\n")[0]
