"""Wait states around the inline-assembly global->LDS copies, checked on the
built library's gfx950 machine code (no GPU needed).

A VMEM instruction may read an SGPR only five wait states after a VALU
instruction wrote it (v_readfirstlane forming a copy's base address, or
v_readlane restoring a spilled SGPR).  The compiler inserts these wait states
for the instructions it generates but not for instructions inside inline
assembly, so every copy block either starts with `s_nop 4` or first copies
its bases with s_mov_b64 (a scalar write needs no wait states before a VMEM
read).  This test disassembles
the code objects of both built libraries and looks, before every
global_load_lds, for a VALU write of its base SGPRs fewer than five wait
states back in program order that no scalar write of them follows.
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_exact_blockwise_amd import build as B

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

_SDST = re.compile(r"^(v_readlane_b32|v_readfirstlane_b32)\s+s(\d+)\b")
_CMP = re.compile(r"^v_cmp\w*\s+s\[(\d+):(\d+)\]")
_CARRY = re.compile(r"^v_\w+\s+v(?:\d+|\[\d+:\d+\]),\s*s\[(\d+):(\d+)\]")
_LDS_DMA = re.compile(r"^global_load_lds_dword\w*\s+v\d+,\s*s\[(\d+):(\d+)\]")


def _instructions(text):
    """(instruction text, function) in address order, per disassembled function."""
    fn = None
    for line in text.split("\n"):
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            fn = m.group(1)
            continue
        ins = line.split("//")[0].strip()
        if ins and fn:
            yield ins, fn


def _sgprs_written_by_valu(ins):
    m = _SDST.match(ins)
    if m:
        return {int(m.group(2))}
    for rx in (_CMP, _CARRY):
        m = rx.match(ins)
        if m:
            return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


_SALU_DST = re.compile(r"^s_(?!cmp|bitcmp|waitcnt|nop|barrier|branch|cbranch|setprio|sleep|sendmsg|endpgm|setpc|swappc|getpc)\w+\s+s(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _sgprs_written_by_salu(ins):
    m = _SALU_DST.match(ins)
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _wait_states(ins):
    m = re.match(r"^s_nop\s+(?:0x)?([0-9a-f]+)", ins)
    if m:
        return int(m.group(1), 16 if "0x" in ins else 10) + 1
    return 1


def find_hazards(text):
    seq = list(_instructions(text))
    found = []
    for i, (ins, fn) in enumerate(seq):
        m = _LDS_DMA.match(ins)
        if not m:
            continue
        need = set(range(int(m.group(1)), int(m.group(2)) + 1))
        states, j = 0, i - 1
        while j >= 0 and states < 5 and seq[j][1] == fn and need:
            if _sgprs_written_by_valu(seq[j][0]) & need:
                found.append((fn, seq[j][0], ins, states))
                break
            need -= _sgprs_written_by_salu(seq[j][0])  # rewritten by a scalar instruction: no wait needed
            states += _wait_states(seq[j][0])
            j -= 1
    return found


def _disassemble(lib, work):
    subprocess.run([f"{LLVM}/llvm-objcopy", "--dump-section", f".hip_fatbin={work}/fat.bin", lib,
                    f"{work}/stripped.so"], check=True, capture_output=True)
    data = open(f"{work}/fat.bin", "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in " + lib
    out = []
    for k, s in enumerate(starts):
        e = starts[k + 1] if k + 1 < len(starts) else len(data)
        open(f"{work}/b{k}.bin", "wb").write(data[s:e])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--input={work}/b{k}.bin", f"--output={work}/b{k}.co", "--unbundle"],
                       check=True, capture_output=True)
        d = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", f"{work}/b{k}.co"], check=True,
                           capture_output=True, text=True)
        out.append(d.stdout)
    return "\n".join(out)


def test_checker_flags_a_close_valu_write():
    text = """0000000000000000 <k>:
\tv_readlane_b32 s19, v253, 56                  // 000000000000: 00000000
\ts_mov_b32 s0, m0                               // 000000000008: 00000000
\ts_mov_b32 m0, s17                              // 00000000000c: 00000000
\ts_nop 0                                        // 000000000010: 00000000
\tglobal_load_lds_dwordx4 v2, s[18:19]           // 000000000014: 00000000
"""
    assert len(find_hazards(text)) == 1
    assert find_hazards(text.replace("s_nop 0 ", "s_nop 4 ")) == []
    assert find_hazards(text.replace("v_readlane_b32 s19", "v_readlane_b32 s21")) == []
    # a scalar copy of the base between the two needs no wait states
    bridged = text.replace("\ts_nop 0 ", "\ts_mov_b64 s[18:19], s[40:41] ")
    assert "s_mov_b64 s[18:19]" in bridged and find_hazards(bridged) == []


@pytest.mark.parametrize("lib", [B.OUT, B.CHECK_OUT], ids=["library", "checking_library"])
def test_no_valu_sgpr_write_shortly_before_a_copy(lib, tmp_path):
    if not os.path.exists(lib):
        pytest.skip(f"{lib} is not built")
    if not shutil.which(f"{LLVM}/llvm-objdump"):
        pytest.skip("llvm-objdump missing")
    text = _disassemble(lib, str(tmp_path))
    assert text.count("global_load_lds") > 100
    hz = find_hazards(text)
    assert hz == [], "\n".join(f"{f}: {w} then {l} after {s} wait states" for f, w, l, s in hz[:10])
