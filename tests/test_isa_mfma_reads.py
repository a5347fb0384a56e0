"""Device-assembly check of the attention kernels (CPU only: hipcc compiles
for gfx950 without a GPU).

The 32x32x16 bf16 MFMA writes its accumulator over many cycles.  A build
of the attention kernel in which the compiler copied accumulators with
VALU moves 12 wait states after the MFMA that produced them gave wrong
values for a few accumulator elements, only on the second wave of each
SIMD, while the same source laid out with no early read was exact.  This
test compiles attention.hip with the library's own flags and checks, along
the straight-line instruction stream after every such MFMA, that no VALU,
LDS or memory instruction reads its result (and no MFMA takes it as an A or
B operand) fewer than MIN_WAIT_STATES wait states later.  A later MFMA
accumulating into the same registers (C operand) is the hardware's own
dependency chain and is not counted."""
import os
import re
import shutil
import subprocess

import pytest

from block_diffusion_draft_vocab_amd import build

MIN_WAIT_STATES = 19  # what a 16-pass XDL result needs before a VALU read
MFMA = "v_mfma_f32_32x32x16_bf16"


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|(?<![\w\[])v(\d+)\b", text):
        if m.group(1):
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _wait_states(line):
    m = re.match(r"s_nop\s+(\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def _reads_and_writes(line):
    """(registers read, registers written) of one vector instruction."""
    op, _, rest = line.partition(" ")
    parts = [p.strip() for p in rest.split(",")]
    if op.startswith(("ds_read", "global_load", "buffer_load", "flat_load")):
        return _regs(",".join(parts[1:])), _regs(parts[0])
    if op.startswith(("ds_write", "global_store", "buffer_store", "flat_store")):
        return _regs(rest), set()
    if op.startswith("v_mfma"):
        return _regs(parts[1]) | _regs(parts[2]), _regs(parts[0])
    if op.startswith("v_"):
        # VOPC writes vcc or an SGPR pair; everything else writes operand 0
        if op.startswith("v_cmp"):
            return _regs(",".join(parts[1:])), set()
        return _regs(",".join(parts[1:])), _regs(parts[0])
    return set(), set()


def _early_reads(asm):
    lines = [ln.strip() for ln in asm.split("\n")]
    found = []
    for i, ln in enumerate(lines):
        if not ln.startswith(MFMA):
            continue
        dst = _regs(ln[len(MFMA):].split(",")[0])
        ws = 0
        for j in range(i + 1, min(len(lines), i + 400)):
            t = lines[j]
            if not t or t.startswith((";", ".", "_")):
                continue
            if t.startswith(("s_branch", "s_endpgm", "s_setpc")):
                break
            reads, writes = _reads_and_writes(t)
            if t.startswith(MFMA):
                # the C operand of a dependent MFMA is waited for by the hardware
                parts = [p.strip() for p in t[len(MFMA):].split(",")]
                reads = _regs(parts[1]) | _regs(parts[2])
            if reads & dst and ws < MIN_WAIT_STATES:
                found.append((ws, ln, t))
            dst -= writes
            if not dst:
                break
            ws += _wait_states(t)
    return found


@pytest.fixture(scope="module")
def attention_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "attention.s"
    cmd = [hipcc, *build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "attention.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out.read_text()


def test_attention_reads_mfma_results_late_enough(attention_asm):
    assert MFMA in attention_asm
    early = _early_reads(attention_asm)
    assert not early, "\n".join(f"{ws} wait states: {m} -> {r}" for ws, m, r in early[:10])


def test_the_check_sees_an_early_read():
    """The scan flags a move of an accumulator 12 wait states after its MFMA
    (the pattern of the bad build) and passes one 48 wait states after."""
    mfma = f"{MFMA} v[2:17], v[70:73], v[74:77], v[2:17]"
    filler = ["v_add_u32_e32 v200, 1, v201"] * 11
    bad = "\n".join([mfma, *filler, "v_mov_b64_e32 v[130:131], v[2:3]"])
    good = "\n".join([mfma, *(filler * 4), "s_nop 3", "v_mov_b64_e32 v[130:131], v[2:3]"])
    assert _early_reads(bad) and not _early_reads(good)
