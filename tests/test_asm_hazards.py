"""Compile the attention kernels to gfx950 assembly and check the MFMA hazards that inline-asm
MFMAs leave to the source (see asm_hazards.py).  Runs on a host without a GPU."""
import os
import re
import subprocess
import sys

import pytest

from asm_hazards import check, kernel_body

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def attn_asm(tmp_path_factory):
    sys.path.insert(0, ROOT)
    from block_causal_chunk_amd import build
    out = tmp_path_factory.mktemp("asm") / "attn_fwd.s"
    cmd = [build.hipcc(), *build.common_flags(), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "attn_fwd.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return out.read_text()


def test_every_attention_kernel_is_hazard_free(attn_asm):
    names = re.findall(r"^(_Z\w*attn_fwd_kernel\w*):", attn_asm, re.M)
    # {d64, d128} x {bf16 out, fp32 out, e4m3 scores, gated bf16, gated e4m3, e4m3 scores + e4m3 V}
    assert len(names) == 12, names
    for n in names:
        found = check(kernel_body(attn_asm, n))
        assert not found, (n, found[:5])
        # and no scratch: a spill inside the key loop would dominate it
        meta = attn_asm[attn_asm.index(n + ":"):]
        assert "scratch_store" not in meta[:meta.index("s_endpgm")], n


def test_checker_finds_a_planted_hazard():
    lines = ["v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
             "s_nop 3",
             "v_accvgpr_read_b32 v8, a3"]
    assert [f[0] for f in check(lines)] == ["RAW"]
    assert check(lines[:1] + ["s_nop 7", "s_nop 3", lines[2]]) == []
    war = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[4:7], v[0:15]", "v_mov_b32 v3, 0"]
    assert [f[0] for f in check(war)] == ["WAR"]
    # a VALU write of an MFMA operand right before it (the constant the compiler rematerialised)
    opnd = ["v_mov_b64_e32 v[8:9], s[98:99]", "v_mfma_f32_32x32x16_bf16 a[0:15], v[6:9], v[20:23], a[0:15]"]
    assert [f[0] for f in check(opnd)] == ["OPND"]
    assert check(opnd[:1] + ["s_nop 1"] + opnd[1:]) == []
