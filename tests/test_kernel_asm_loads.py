"""The attention kernel loads Q (and its rotation rows) with inline-asm
global loads so that their wait does not also wait for the direct-to-LDS tile
stream, and reads V for its conversion with inline-asm transposing LDS reads;
the compiler does not know such a load is in flight, so it must not read,
write or reload any of its destination registers before the explicit wait
(vmcnt for the global loads, lgkmcnt for the LDS reads).  This test compiles csrc/attention.hip for gfx950 (our own
source), and checks every attention kernel's prologue on every control-flow
path (no GPU).  A kernel whose register pressure made the compiler copy or
reuse an in-flight destination faulted the GPU with an illegal address."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "kv_cache_attention_ring_amd")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _blocks(lines):
    bl, cur = [], {"label": None, "ins": []}
    for line in lines:
        t = line.strip()
        m = re.match(r"^(\.LBB\w+):", t)
        if m:
            bl.append(cur)
            cur = {"label": m.group(1), "ins": []}
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        cur["ins"].append(t)
        op = t.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm"):
            bl.append(cur)
            cur = {"label": None, "ins": []}
    bl.append(cur)
    return [b for b in bl if b["ins"] or b["label"]]


def audit(lines):
    """Violations on any path from entry to the first s_waitcnt vmcnt
    (s_cbranch_execnz taken, s_cbranch_execz not: all lanes are active)."""
    bl = _blocks(lines)
    idx = {b["label"]: i for i, b in enumerate(bl) if b["label"]}
    succ = []
    for i, b in enumerate(bl):
        last = b["ins"][-1] if b["ins"] else ""
        op = last.split()[0] if last else ""
        nxt = [i + 1] if i + 1 < len(bl) else []
        if op in ("s_branch", "s_cbranch_execnz"):
            succ.append([idx[last.split()[1]]])
        elif op == "s_cbranch_execz":
            succ.append(nxt)
        elif op.startswith("s_cbranch"):
            succ.append([idx[last.split()[1]]] + nxt)
        elif op == "s_endpgm":
            succ.append([])
        else:
            succ.append(nxt)
    IN, bad, work = {0: frozenset()}, set(), [0]
    while work:
        i = work.pop()
        infl, waited = set(IN[i]), False
        for t in bl[i]["ins"]:
            op = t.split()[0]
            if op == "s_waitcnt" and "vmcnt" in t:
                waited = True
                break
            toks = [x.rstrip(",") for x in t.split()[1:]]
            if op == "global_load_dwordx4":
                if _regs(toks[0]) & infl or _regs(toks[1]) & infl:
                    bad.add(t)
                infl |= _regs(toks[0])
                continue
            if any(_regs(x) & infl for x in toks):
                bad.add(t)
        if waited:
            continue
        for j in succ[i]:
            new = frozenset(IN.get(j, frozenset()) | infl)
            if j not in IN or new != IN[j]:
                IN[j] = new
                work.append(j)
    return sorted(bad)


def _succ(bl):
    idx = {b["label"]: i for i, b in enumerate(bl) if b["label"]}
    succ = []
    for i, b in enumerate(bl):
        last = b["ins"][-1] if b["ins"] else ""
        op = last.split()[0] if last else ""
        nxt = [i + 1] if i + 1 < len(bl) else []
        if op == "s_branch":
            succ.append([idx[last.split()[1]]])
        elif op.startswith("s_cbranch"):
            succ.append([idx[last.split()[1]]] + nxt)
        elif op == "s_endpgm":
            succ.append([])
        else:
            succ.append(nxt)
    return succ


def audit_lds_transpose(lines):
    """The transposing LDS reads (ds_read_b64_tr_b8) are issued from inline
    asm too: on every path through the whole kernel, loops included, no
    instruction may touch a read's destination before an s_waitcnt
    lgkmcnt(0)."""
    bl = _blocks(lines)
    succ = _succ(bl)
    IN, bad, work = {0: frozenset()}, set(), [0]
    while work:
        i = work.pop()
        infl = set(IN[i])
        for t in bl[i]["ins"]:
            op = t.split()[0]
            if op == "s_waitcnt" and "lgkmcnt(0)" in t:
                infl.clear()
                continue
            toks = [x.rstrip(",") for x in t.split()[1:]]
            if op == "ds_read_b64_tr_b8":
                if _regs(toks[0]) & infl or _regs(toks[1]) & infl:
                    bad.add(t)
                infl |= _regs(toks[0])
                continue
            if any(_regs(x) & infl for x in toks):
                bad.add(t)
        for j in succ[i]:
            new = frozenset(IN.get(j, frozenset()) | infl)
            if j not in IN or new != IN[j]:
                IN[j] = new
                work.append(j)
    return sorted(bad)


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_attention_prologue_keeps_asm_load_destinations(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    out = str(tmp_path / "attention.s")
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(PKG, "csrc", "attention.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    s = open(out).read()
    names = re.findall(r"^(_ZN3kvr12_GLOBAL__N_1\w*attn\w*kernel\w+):", s, flags=re.M)
    assert len(names) >= 8, names
    for name in names:
        i = s.index(name + ":")
        body = s[i:s.index(".Lfunc_end", i)].split("\n")
        assert any("global_load_dwordx4" in l for l in body), name
        bad = audit(body)
        assert not bad, f"{name}: {bad[:3]}"
        assert any("ds_read_b64_tr_b8" in l for l in body), name
        bad = audit_lds_transpose(body)
        assert not bad, f"{name}: transposing read destination touched before its wait: {bad[:3]}"


def test_lds_audit_flags_a_use_before_the_wait_around_a_loop():
    lines = [".LBB0_1:",
             "\tds_read_b64_tr_b8 v[4:5], v2",
             "\tv_add_u32_e32 v9, v10, v11",
             "\ts_cbranch_scc1 .LBB0_1",
             "\tv_mov_b32_e32 v6, v4",
             "\ts_waitcnt lgkmcnt(0)",
             "\ts_endpgm"]
    # the use after the loop, and the read issued again around the loop over
    # its own destination while the first is in flight
    bad = audit_lds_transpose(lines)
    assert len(bad) == 2 and any(b.startswith("v_mov") for b in bad) and \
        any(b.startswith("ds_read_b64_tr_b8") for b in bad)
    ok = [".LBB0_1:", "\tds_read_b64_tr_b8 v[4:5], v2", "\ts_waitcnt lgkmcnt(0)",
          "\tv_mov_b32_e32 v6, v4", "\ts_cbranch_scc1 .LBB0_1", "\ts_endpgm"]
    assert audit_lds_transpose(ok) == []


def test_audit_flags_a_copied_in_flight_destination():
    # a load followed by a copy of its destination before the wait, and a
    # reuse of a destination as the next address: both flagged
    lines = ["\tglobal_load_dwordx4 v[4:7], v[2:3], off",
             "\tv_accvgpr_write_b32 a0, v4",
             "\tglobal_load_dwordx4 v[8:11], v[4:5], off",
             "\ts_waitcnt vmcnt(0)"]
    assert len(audit(lines)) == 2
    ok = ["\tglobal_load_dwordx4 v[4:7], v[4:5], off", "\tv_add_u32_e32 v9, v10, v11",
          "\ts_waitcnt vmcnt(0)", "\tv_accvgpr_write_b32 a0, v4"]
    assert audit(ok) == []
