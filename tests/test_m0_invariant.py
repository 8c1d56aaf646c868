"""The LDS-DMA copies of the decode and prefill kernels set the m0 register in inline assembly, which the
compiler does not track: each copy is the three-instruction block `s_mov_b32 m0, sN; s_nop 0;
global_load_lds_dwordx4`.  That is sound only while nothing the compiler emits in those kernels reads or
writes m0 (a compiler-placed m0 value live across a copy block would be overwritten).  This test compiles
the two kernel sources to gfx950 assembly with the library's flags and checks that invariant: every m0
mention is one of the copy blocks' writes, each write is followed by its copy, and no instruction that
reads m0 implicitly (relative register moves, GPR indexing, messages, LDS DMA by buffer loads, GWS,
append/consume, interpolation) appears.  CPU only; about half a minute.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_15_amd", "csrc")
sys.path.insert(0, os.path.join(ROOT, "decode_attention_15_amd"))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
IMPLICIT_M0 = re.compile(r"\b(v_movrel\w*|s_movrel\w*|s_set_gpr_idx\w*|s_sendmsg\w*|buffer_load_\w*lds\w*|"
                         r"buffer_store_lds\w*|ds_gws\w*|ds_append|ds_consume|ds_ordered_count|v_interp\w*|"
                         r"s_ttracedata)\b")


def _device_asm(src, tmp_path):
    import build
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [HIPCC, *build.COMMON, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"hipcc failed:\n{' '.join(cmd)}\n{r.stderr[-3000:]}")
    with open(out) as f:
        return f.read().splitlines()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("name", ["kvq_decode.hip", "kvq_prefill.hip"])
def test_m0_is_written_only_by_the_copy_blocks(name, tmp_path):
    lines = [ln.split(";")[0].strip() for ln in _device_asm(os.path.join(CSRC, name), tmp_path)]
    ins = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
    writes = copies = 0
    for i, ln in enumerate(ins):
        assert not IMPLICIT_M0.search(ln), f"{name}: an instruction that reads m0 implicitly: {ln}"
        if ln.startswith("global_load_lds_dwordx4"):
            copies += 1
            assert i >= 2 and re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 2]) and ins[i - 1] == "s_nop 0", \
                f"{name}: a copy not preceded by its m0 write: {ins[i - 2:i + 1]}"
        if re.search(r"\bm0\b", ln):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"{name}: m0 used outside a copy block: {ln}"
            assert i + 2 < len(ins) and ins[i + 2].startswith("global_load_lds_dwordx4"), \
                f"{name}: an m0 write not followed by its copy: {ins[i:i + 3]}"
            writes += 1
    assert copies > 0 and writes == copies, (name, writes, copies)
