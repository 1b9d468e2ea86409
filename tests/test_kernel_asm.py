"""Checks on the gfx950 assembly of the library's kernels (CPU only: hipcc cross-compiles).

A vector memory store of more than 8 bytes of data (dwordx3 / dwordx4) keeps reading its
data registers for a while after it issues.  A VALU instruction that writes one of those
registers in the next slot changed what some lanes of such a store wrote on MI355X
(nondeterministic, wrong kept softmax terms), and the compiler does not put a wait state
there by itself.  Every such store must be followed by at least two wait states (other
instructions or an s_nop) before a VALU write of its data registers.
"""

import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    # by file path: importing the package would load the library being checked
    spec = importlib.util.spec_from_file_location(
        "grpo_build", os.path.join(ROOT, "grpo_loss_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


WIDE_STORE = re.compile(r"^(buffer|global|flat|scratch)_store_dwordx[34]\s+(.*)$")
REG_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
VALU_DST = re.compile(r"^v_\S+\s+([va])\[?(\d+)(?::(\d+))?")
NOP = re.compile(r"^s_nop\s+(\d+)")
NEEDED_STATES = 2


def wide_store_hazards(asm: str):
    """(function, store, offending instruction) for each wide store whose data registers a
    VALU instruction writes within NEEDED_STATES wait states."""
    out = []
    func = "?"
    lines = []
    for raw in asm.split("\n"):
        s = raw.split(";")[0].strip()
        m = re.match(r"^(_Z\w+):", s)
        if m:
            func = m.group(1)
            continue
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        lines.append((func, s))
    for i, (fn, s) in enumerate(lines):
        m = WIDE_STORE.match(s)
        if not m:
            continue
        # buffer stores take the data first; global, flat and scratch stores the address
        ops = [o.strip() for o in m.group(2).split(",")]
        r = REG_RANGE.match(ops[0] if m.group(1) == "buffer" else ops[1])
        assert r, s
        cls, lo, hi = r.group(1), int(r.group(2)), int(r.group(3))
        states = 0
        for fn2, nxt in lines[i + 1:i + 1 + NEEDED_STATES]:
            if fn2 != fn or states >= NEEDED_STATES:
                break
            n = NOP.match(nxt)
            if n:
                states += int(n.group(1)) + 1
                continue
            d = VALU_DST.match(nxt)
            if d and d.group(1) == cls:
                a = int(d.group(2))
                b = int(d.group(3) or a)
                if a <= hi and b >= lo:
                    out.append((fn, s, nxt))
                    break
            states += 1
    return out


def test_scanner_flags_a_planted_hazard():
    asm = "\n".join([
        "_Zk:",
        "\tbuffer_store_dwordx4 v[132:135], v252, s[0:3], s84 offen",
        "\tv_fma_f32 v132, v114, s33, -v131",
        "\tbuffer_store_dwordx4 v[10:13], v252, s[0:3], s84 offen",
        "\ts_nop 1",
        "\tv_mov_b32_e32 v10, 0",
        "\tglobal_store_dwordx4 v[0:1], v[20:23], off",
        "\tv_add_f32_e32 v5, v6, v7",
        "\tv_add_f32_e32 v21, v6, v7",
        "\tbuffer_store_dwordx2 v[40:41], v252, s[0:3], 0 offen",
        "\tv_mov_b32_e32 v40, 0",
    ])
    hz = wide_store_hazards(asm)
    assert [h[2] for h in hz] == ["v_fma_f32 v132, v114, s33, -v131",
                                  "v_add_f32_e32 v21, v6, v7"]


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None,
                    reason="hipcc not available")
def test_no_wide_store_data_hazard(tmp_path):
    b = _build_module()
    bad = []
    for src in b.sources():
        out = tmp_path / (src + ".s")
        cmd = [b.HIPCC, *b.COMMON, *b.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(b.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        asm = out.read_text()
        assert "_Z" in asm
        bad += [(src, *h) for h in wide_store_hazards(asm)]
    assert not bad, "\n".join(f"{s}: {fn[:60]}: {st} -> {nx}" for s, fn, st, nx in bad[:20])
