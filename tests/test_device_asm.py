"""Generated gfx950 code of the kernels that stage tiles with direct-to-LDS
copies (CPU only: hipcc cross-compiles the device code to assembly here).

The copy writes M0 inside an inline-assembly statement, and the compiler
does not accept M0 as a clobber, so nothing else in these kernels may keep a
value in M0 or use it implicitly.  Every write of M0 must be the copy's own
sequence (s_mov_b32 m0, then one wait state, then the LDS-bound load), and
every instruction that reads M0 implicitly must be that load.
"""
import os
import re
import subprocess

import pytest

from sequence_approximate_attention_amd import build as B

SOURCES = ["attn_bf16.hip", "score_bf16.hip"]

# Instructions that read M0 without naming it.
IMPLICIT_M0 = re.compile(r"^(s_sendmsg\w*|s_movrel\w*|v_movrel\w*|v_interp\w*|ds_gws\w*|ds_append|ds_consume"
                         r"|ds_\w+_addtid\w*|s_ttracedata|lds_\w+)$")


def instructions(asm_text):
    out = []
    for line in asm_text.splitlines():
        s = line.strip()
        if not s or s[0] in ";." or s.endswith(":") or not line.startswith(("\t", " ")):
            continue
        s = s.split(";")[0].strip()
        if s and re.match(r"^[a-z_][a-z0-9_]*", s):
            out.append(s)
    return out


def lds_bound_load(ins):
    op = ins.split()[0]
    return op.startswith(("buffer_load", "global_load")) and re.search(r"\blds\b", ins) is not None


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    res = {}
    for src in SOURCES:
        out = os.path.join(d, src.replace(".hip", ".s"))
        cmd = [hipcc, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-S", "--cuda-device-only",
               os.path.join(B.CSRC, src), "-o", out, *B.DEVICE_FLAGS, *B.SOURCE_FLAGS.get(src, [])]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        res[src] = instructions(open(out).read())
    return res


def m0_violations(ins):
    """Instructions that write or read M0 outside the copy's own sequence."""
    bad = []
    for i, s in enumerate(ins):
        op = s.split()[0]
        operands = s[len(op):]
        if re.search(r"\bm0\b", operands):
            ok = (op == "s_mov_b32" and re.match(r"^\s*m0,\s*s\d+$", operands) is not None
                  and i + 2 < len(ins) and ins[i + 1] == "s_nop 0" and lds_bound_load(ins[i + 2]))
            if not ok:
                bad.append(s)
        elif lds_bound_load(s) or IMPLICIT_M0.match(op):
            ok = i >= 2 and ins[i - 1] == "s_nop 0" and re.match(r"^s_mov_b32\s+m0,\s*s\d+$", ins[i - 2])
            if not ok:
                bad.append(s)
    return bad


def test_the_check_flags_stray_m0_uses():
    copy = ["s_mov_b32 m0, s49", "s_nop 0", "buffer_load_dwordx4 v133, s[16:19], s63 offen lds"]
    assert m0_violations(["v_add_u32_e32 v1, v2, v3"] + copy + ["s_barrier"]) == []
    assert m0_violations(["s_mov_b32 m0, s4", "v_add_u32_e32 v1, v2, v3"] + copy) == ["s_mov_b32 m0, s4"]
    assert m0_violations(copy + ["s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)"]) == ["s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)"]
    assert m0_violations(["s_mov_b32 s0, m0"] + copy) == ["s_mov_b32 s0, m0"]
    stray = "buffer_load_dword v2, s[16:19], s63 offen lds"
    assert m0_violations(copy + ["s_nop 0", stray]) == [stray]


@pytest.mark.parametrize("src", SOURCES)
def test_m0_is_only_the_tile_copy_address(device_asm, src):
    ins = device_asm[src]
    assert m0_violations(ins) == [], f"{src}: M0 used outside the tile copies"
    n_copies = sum(1 for s in ins if lds_bound_load(s))
    assert n_copies > 0, f"{src}: no tile copies found"
