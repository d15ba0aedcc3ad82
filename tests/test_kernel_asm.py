"""Static checks on the gfx950 assembly of the split attention kernel (no GPU).

The split kernel writes some of its MFMAs as inline asm (the QK chain keeps
its accumulator in VGPRs that way).  The compiler's hazard recognizer does
not know what an asm statement contains, so it cannot insert the two wait
states gfx950 needs between a VALU instruction that writes a VGPR and an
MFMA that reads it; the kernel has to provide them itself (the 8-bit path
converts each fragment two MFMAs ahead and puts an s_nop in front of the
first).  A VALU write that lands too close makes the MFMA read a stale
operand, which shows up only as occasional wrong results on the device.
This test compiles decode_v3.hip to assembly with the build's flags and
checks every asm MFMA of every k_split instance.
"""

import os
import re
import shutil
import subprocess

import pytest

from head_latent_attention_16_amd import build as B

HIPCC = B.HIPCC
WAIT_STATES = 2   # VALU write of a VGPR -> MFMA reading it


def _have_hipcc():
    return os.path.isfile(HIPCC) and os.access(HIPCC, os.X_OK) or shutil.which(HIPCC) is not None


def _regs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _operands(inst):
    parts = inst.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def _hazards(asm_text, kernel):
    start = asm_text.index(kernel + ":") + len(kernel) + 1   # past the function's own label
    end = asm_text.index(".Lfunc_end", start)
    # (text, is_asm, is_label) per line that issues or breaks straight-line code
    items = []
    in_asm = False
    for line in asm_text[start:end].split("\n"):
        t = line.split(";", 1)[0].strip() if not line.strip().startswith(";;#ASM") else line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith("."):
            continue
        if t.endswith(":"):
            items.append((t, False, True))
            continue
        items.append((t, in_asm, False))
    found = []
    for k, (inst, is_asm, _) in enumerate(items):
        if not (is_asm and inst.startswith("v_mfma")):
            continue
        src = set().union(*[_regs(o) for o in _operands(inst)[1:]])
        waits = 0
        j = k - 1
        while j >= 0 and waits < WAIT_STATES:
            prev, _, is_label = items[j]
            if is_label:
                found.append(f"{inst}: fewer than {WAIT_STATES} wait states to the start of its block")
                break
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
            else:
                ops = _operands(prev)
                if prev.startswith("v_") and not prev.startswith("v_mfma") and ops and _regs(ops[0]) & src:
                    found.append(f"{prev} -> {inst} ({waits} wait states)")
                    break
                waits += 1
            j -= 1
    return found


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_asm_mfma_operands_have_their_wait_states(tmp_path):
    out = tmp_path / "decode_v3.s"
    cmd = [HIPCC, *B.COMMON, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(B.CSRC, "decode_v3.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    kernels = sorted(set(re.findall(r"^(_Z\w*k_split\w*):", text, re.M)))
    assert len(kernels) == 6, kernels   # SCAN x {16-bit, paged, 8-bit}
    n_asm = 0
    for k in kernels:
        body = text[text.index(k + ":"):text.index(".Lfunc_end", text.index(k + ":"))]
        n_asm += len(re.findall(r";;#ASMSTART\s*\n\s*v_mfma", body))
        bad = _hazards(text, k)
        assert not bad, (k, bad[:10])
    assert n_asm > 0


def test_hazard_scan_catches_a_planted_write():
    """The scanner itself: a VALU write right before an asm MFMA is reported,
    one two instructions earlier is not, and an s_nop counts its wait states."""
    def kern(lines):
        return "_Zk:\n" + "\n".join(lines) + "\n.Lfunc_end0:\n"
    mfma = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]", ";;#ASMEND"]
    assert _hazards(kern(["v_mov_b32 v21, 0"] + mfma), "_Zk")
    assert _hazards(kern(["v_mov_b32 v25, 0", "s_mov_b32 s0, 0"] + mfma), "_Zk")
    assert not _hazards(kern(["v_mov_b32 v21, 0", "s_mov_b32 s0, 0", "s_mov_b32 s1, 0"] + mfma), "_Zk")
    assert not _hazards(kern(["v_mov_b32 v21, 0", "s_nop 1"] + mfma), "_Zk")
    assert not _hazards(kern(["v_mov_b32 v40, 0"] + mfma), "_Zk")
    assert _hazards(kern(["label0:"] + mfma), "_Zk")
