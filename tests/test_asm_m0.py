"""The direct-to-LDS loads of the GEMM kernels set M0 (the LDS destination
base) in inline asm, which the compiler does not see as a write of that
register: they are correct only while no instruction the compiler itself
emits in the same kernels reads or writes M0.  This compiles every source
holding such loads for gfx950 to assembly (device code only, the library's
own flags) and checks that every instruction naming m0 lies inside an
inline-asm block, and that each source does hold such blocks."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from dropless_moe_expert_amd import build as b

SOURCES = ["gg_bf16.hip", "gg_fwd_mx.hip", "gg_mx4.hip", "route_fused.hip"]
M0 = re.compile(r"\bm0\b")


def _assemble(src: str, out: str) -> str:
    cmd = [b._hipcc()] + b.CFLAGS + b.SOURCE_FLAGS.get(src, []) + [
        "--cuda-device-only", "-S", os.path.join(b.CSRC, src), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    with open(out) as f:
        return f.read()


def m0_uses(asm: str):
    """(instructions naming m0 inside inline asm, those outside it)."""
    inside, outside = [], []
    in_asm = False
    for n, line in enumerate(asm.splitlines(), 1):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = s.split(";", 1)[0].strip()
        if not code or code.startswith(".") or code.endswith(":"):
            continue
        if M0.search(code):
            (inside if in_asm else outside).append((n, code))
    return inside, outside


def test_m0_parser_on_a_sample():
    asm = "\n".join([
        "k:", "\ts_mov_b32 s0, 1", "\t;;#ASMSTART", "\ts_mov_b32 m0, s14",
        "\tglobal_load_lds_dwordx4 v2, s[4:5]", "\t;;#ASMEND",
        "\ts_mov_b32 m0, -1 ; compiler's own", "\t; a comment naming m0",
        "\t.set m0_like, 1", "\ts_endpgm"])
    inside, outside = m0_uses(asm)
    assert [c for _, c in inside] == ["s_mov_b32 m0, s14"]
    assert [c for _, c in outside] == ["s_mov_b32 m0, -1"]


@pytest.mark.timeout(900)
def test_compiler_leaves_m0_to_the_inline_asm(tmp_path):
    outs = {src: str(tmp_path / (src + ".s")) for src in SOURCES}
    with ThreadPoolExecutor(max_workers=4) as ex:
        asm = dict(zip(SOURCES, ex.map(lambda s: _assemble(s, outs[s]), SOURCES)))
    for src, text in asm.items():
        inside, outside = m0_uses(text)
        assert inside, f"{src}: no inline-asm write of m0 found"
        assert not outside, f"{src}: compiler-emitted instructions name m0: {outside[:5]}"
