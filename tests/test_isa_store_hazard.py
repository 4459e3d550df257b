"""Store-data hazard scan of the gfx950 code of every kernel (CPU only).

A vector memory store of more than 64 bits reads its upper data registers
after it issues, so a VALU write of those registers needs wait states after
it; the compiler inserts them.  On one build of the tall RowNorm kernel, a
16-byte buffer store closed a conditional block and the join block began by
writing the store's data registers with no wait states between them: the
store's last lanes wrote the new value into W.  That kernel now stores 8
bytes at a time and follows each store with `s_nop 2`.  This test compiles
every HIP source to gfx950 assembly, as the build does, and checks that no
VALU instruction writes the data registers of a store of more than 8 bytes
within two wait states of it, following fall-through across block labels and
the targets of branches.  A compiler change that re-opens the pattern fails
here instead of corrupting weights on the GPU.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_aware_optimizer_periodic_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
WINDOW = 2          # wait states after a store in which its data may not be written

STORE = re.compile(r"^(global|buffer|flat)_store_(dwordx3|dwordx4|b96|b128)\s+(.*)$")


def regs(tok):
    """VGPR / AGPR numbers named by one operand, as ('v', n) / ('a', n)."""
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def functions(asm):
    """Instruction lists per function, with the label positions of each."""
    out = {}
    name, ins, labels = None, [], {}
    for raw in asm.splitlines():
        line = raw.split(";")[0].rstrip()
        s = line.strip()
        if not s:
            continue
        if re.match(r"^[A-Za-z_.$][\w.$]*:$", s) and not line.startswith((" ", "\t")):
            lab = s[:-1]
            if lab.startswith(".L"):
                labels[lab] = len(ins)
            else:
                if name is not None:
                    out[name] = (ins, labels)
                name, ins, labels = lab, [], {}
            continue
        if s.startswith("."):
            continue
        if name is not None:
            ins.append(s)
    if name is not None:
        out[name] = (ins, labels)
    return out


def wait_states(op):
    m = re.match(r"s_nop\s+(\d+)", op)
    return int(m.group(1)) + 1 if m else 1


def followers(ins, labels, start, budget, seen=None):
    """Instructions that may issue within `budget` wait states after ins[start]."""
    seen = set() if seen is None else seen
    out = []
    k = start + 1
    while budget > 0 and k < len(ins):
        if (k, budget) in seen:
            break
        seen.add((k, budget))
        op = ins[k]
        out.append(op)
        budget -= wait_states(op)
        if op.startswith("s_endpgm"):
            break
        m = re.match(r"s_(c?)branch\w*\s+(\.L\w+)", op)
        if m and m.group(2) in labels:
            out += followers(ins, labels, labels[m.group(2)] - 1, budget, seen)
            if not m.group(1):
                break                       # unconditional: no fall-through
        k += 1
    return out


def scan(asm):
    problems, checked = [], 0
    for fn, (ins, labels) in functions(asm).items():
        for k, op in enumerate(ins):
            m = STORE.match(op)
            if not m:
                continue
            ops = [o.strip() for o in m.group(3).split(",")]
            data = regs(ops[0]) if m.group(1) == "buffer" else regs(ops[1])
            checked += 1
            for nxt in followers(ins, labels, k, WINDOW):
                if not nxt.startswith("v_"):
                    continue
                parts = nxt.split(None, 1)
                if len(parts) < 2:
                    continue
                dst = regs(parts[1].split(",")[0])
                if dst & data:
                    problems.append(f"{fn}: '{op}' then '{nxt}'")
    return problems, checked


def test_scanner_flags_the_pattern():
    """The scan finds a write of a store's data across a block join, and
    accepts the same code with the nop guard between them."""
    bad = """kern:
\tbuffer_store_dwordx4 v[4:7], v1, s[0:3], s6 offen
.LBB0_2:
\tv_mov_b64_e32 v[6:7], s[8:9]
\ts_endpgm
"""
    good = bad.replace("offen\n", "offen\n\ts_nop 2\n")
    branch = """kern:
\tglobal_store_dwordx4 v[0:1], v[8:11], off
\ts_cbranch_scc1 .LBB0_4
\ts_endpgm
.LBB0_4:
\tv_add_u32_e32 v10, v1, v2
\ts_endpgm
"""
    assert scan(bad)[0] and not scan(good)[0] and scan(branch)[0]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_store_data_overwritten_within_two_wait_states(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    problems, checked = scan(out.read_text())
    print(f"{src}: {checked} stores of more than 8 bytes checked")
    assert not problems, "\n".join(problems[:10])
