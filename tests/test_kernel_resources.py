"""Resource guard for the gfx950 kernels (no GPU needed): every kernel of the
library compiles with no scratch memory and no vector-register spills.  A
spill in the decode loop puts a wait for all outstanding memory operations
into every tile, so a regression must fail here rather than show up only as a
slower benchmark.  (Scalar-register spills are allowed: they go to lanes of
vector registers, not to memory.)  The compiler's own resource-usage report
is parsed; the 128-head FP8 decode kernels must also keep occupancy 1 with
the whole register file (they are written for it).

The score products of the FP8 decode are issued as inline assembly, which the
compiler's hazard recognizer does not look into, so the device assembly is
also checked for the data hazards around those matrix instructions that the
hardware leaves to software (a VALU write of an operand just before the
instruction; a read or write of its result while it is still in flight)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_mla_attention_decode_amd import build as B


def _report(src, asm_dir):
    asm = os.path.join(asm_dir, os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.compile_flags(), "--cuda-device-only", "-S", "-o", asm,
           "-Rpass-analysis=kernel-resource-usage", src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {"__asm__": open(asm).read()}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\w+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return kernels


@pytest.fixture(scope="module")
def reports(tmp_path_factory):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(max_workers=3) as ex:
        return dict(zip(B.sources(), ex.map(lambda s: _report(s, d), B.sources())))


def test_no_kernel_uses_scratch_or_spills(reports):
    seen = 0
    for src, kernels in reports.items():
        for name, r in kernels.items():
            if "kernel" not in name or name == "__asm__":
                continue
            seen += 1
            assert r.get("ScratchSize") == "0", (os.path.basename(src), name, r)
            assert r.get("VGPRs Spill") == "0", (os.path.basename(src), name, r)
            assert r.get("Dynamic Stack") == "False", (os.path.basename(src), name, r)
    assert seen >= 10


def test_h128_decode_keeps_the_whole_register_file(reports):
    names = {n: r for k in reports.values() for n, r in k.items() if n != "__asm__"}
    dec = {n: r for n, r in names.items() if "decode_fp8_h128_kernel" in n}
    # 656-byte rows: flat / paged address x sparse / dense x 128 / 64 heads;
    # V4, V4.1, V4.1 with an FP4 extra cache and bf16 rows: sparse x 128 / 64 heads
    assert len(dec) == 16
    for n, r in dec.items():
        h64 = re.search(r"ILb[01]ELb[01]ELb([01])E", n).group(1) == "1"
        # O^T for 128 dims x 128 heads fills the 256 AGPRs; with 64 heads half of it
        assert r["Occupancy"] == "1" and int(r["AGPRs"]) >= (128 if h64 else 256), (n, r)
    for needle in ("combine_packed_kernel", "gather_h128_kernel", "indexer_score_kernel",
                   "indexer_topk_kernel", "sched_parallel_kernel", "sched_flat_kernel", "sched_kernel"):
        assert any(needle in n for n in names), needle


# ---- matrix-instruction hazards around inline assembly ---------------------
# Software-resolved dependencies of CDNA3/CDNA4 matrix instructions (the
# "required wait states" tables of the MI300 instruction set reference):
# a VALU write of a VGPR followed by an MFMA that reads it needs 2 wait
# states; an XDL MFMA's result read (or overwritten) by a non-matrix
# instruction needs up to 19 for a 16-pass op (11 for the 8-pass 32x32x16
# bf16 op; 19 is the bound checked).  MFMA-to-MFMA chaining through SrcC is
# interlocked and not checked.
VALU_TO_MFMA = 2
MFMA_TO_OTHER = 19

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        lo = int(m.group(2) if m.group(2) is not None else m.group(4))
        hi = int(m.group(3)) if m.group(3) is not None else lo
        out.update((m.group(1), i) for i in range(lo, hi + 1))
    return out


def _functions(asm):
    """{symbol: [lines]} for every function body in a device assembly file."""
    funcs, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is not None and line.startswith(".Lfunc_end"):
            cur = None
        elif cur is not None:
            cur.append(line)
    return funcs


def _program(lines):
    """Instructions of one function with its control-flow graph: (ins, succ,
    pred, inline, cond).  ins[i] = (mnemonic, operands, wait states it counts
    for); cond[i] names the wave-uniform value a conditional branch tests when
    the instruction before it is `s_and_b64 vcc, exec, X` (the form a
    wave-uniform `if` takes), so that branches on the same X can be followed
    consistently."""
    ins, labels, inline, pending, in_asm = [], {}, [], [], False
    for raw in lines:
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t or t.startswith("."):
            m = re.match(r"^(\.L\w+):", t)
            if m:
                pending.append(m.group(1))
            continue
        op, _, rest = t.partition(" ")
        for lab in pending:
            labels[lab] = len(ins)
        pending = []
        ws = int(rest.strip()) + 1 if op == "s_nop" else 1
        ins.append((op, rest.strip(), ws))
        inline.append(in_asm)
    n = len(ins)
    succ = [[] for _ in range(n)]
    cond = [None] * n
    for i, (op, rest, _) in enumerate(ins):
        tgt = rest.split(",")[0].strip()
        if op == "s_branch":
            succ[i] = [labels[tgt]] if tgt in labels else []
        elif op.startswith("s_cbranch"):
            succ[i] = ([labels[tgt]] if tgt in labels else []) + ([i + 1] if i + 1 < n else [])
            if op in ("s_cbranch_vccnz", "s_cbranch_vccz") and i > 0 and ins[i - 1][0] == "s_and_b64":
                ops = [o.strip() for o in ins[i - 1][1].split(",")]
                if len(ops) == 3 and ops[0] == "vcc" and "exec" in ops[1:]:
                    cond[i] = ops[2] if ops[1] == "exec" else ops[1]
        elif op in ("s_endpgm", "s_setpc_b64", "s_trap"):
            succ[i] = []
        elif i + 1 < n:
            succ[i] = [i + 1]
    pred = [[] for _ in range(n)]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return ins, succ, pred, inline, cond, labels


def _dst_src(rest):
    ops = [o.strip() for o in rest.split(",")]
    return _regs(ops[0]) if ops else set(), set().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else set()


_SREG = re.compile(r"\bs(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _sregs(text):
    out = set()
    for m in _SREG.finditer(text):
        lo = int(m.group(1) if m.group(1) is not None else m.group(3))
        hi = int(m.group(2)) if m.group(2) is not None else lo
        out.update(range(lo, hi + 1))
    return out


def _hazards(lines):
    ins, succ, pred, inline, cond, labels = _program(lines)

    def edge(b, to):
        """Value of branch b's tested X (nonzero?) on the edge b -> to, or None."""
        if cond[b] is None or len(set(succ[b])) < 2:
            return None
        taken = to != b + 1
        return taken if ins[b][0] == "s_cbranch_vccnz" else not taken

    def writes(j, key):
        op, rest, _ = ins[j]
        return op.startswith("s_") and bool(_sregs(rest.split(",")[0]) & _sregs(key))

    def guard(i):
        """Assumptions under which instruction i runs: the uniform branch that
        leads to its straight-line block, if any."""
        j = i
        while len(pred[j]) == 1:
            p = pred[j][0]
            v = edge(p, j)
            if v is not None:
                return frozenset({(cond[p], v)})
            if p != j - 1:
                break
            j = p
        return frozenset()

    def consistent(assume, key, v):
        return (key, not v) not in assume

    found = []
    for i, (op, rest, _) in enumerate(ins):
        if not (inline[i] and op.startswith("v_mfma")):
            continue
        dst, src = _dst_src(rest)
        g = guard(i)
        # backwards: a VALU write of a source operand fewer than 2 wait states before
        stack, seen = [(p, 0, g, i) for p in pred[i]], set()
        while stack:
            j, ws, assume, came = stack.pop()
            v = edge(j, came)
            if v is not None:
                if not consistent(assume, cond[j], v):
                    continue
                assume = assume | {(cond[j], v)}
            if (j, ws, assume) in seen or ws >= VALU_TO_MFMA:
                continue
            seen.add((j, ws, assume))
            jop, jrest, jws = ins[j]
            if jop.startswith("v_") and not jop.startswith("v_mfma") and _dst_src(jrest)[0] & src:
                found.append(f"{jop} {jrest} -> {op} {rest} ({ws} wait states)")
            assume = frozenset(a for a in assume if not writes(j, a[0]))
            stack.extend((p, ws + jws, assume, j) for p in pred[j])
        # forwards: a non-matrix instruction touching the result while in flight
        stack, seen = [(s_, 0, g, i) for s_ in succ[i]], set()
        while stack:
            j, ws, assume, came = stack.pop()
            v = edge(came, j)
            if v is not None:
                if not consistent(assume, cond[came], v):
                    continue
                assume = assume | {(cond[came], v)}
            if (j, ws, assume) in seen or ws >= MFMA_TO_OTHER:
                continue
            seen.add((j, ws, assume))
            jop, jrest, jws = ins[j]
            if not jop.startswith(("v_mfma", "s_")) and _regs(jrest) & dst:
                found.append(f"{op} {rest} -> {jop} {jrest} ({ws} wait states)")
                continue
            assume = frozenset(a for a in assume if not writes(j, a[0]))
            stack.extend((s_, ws + jws, assume, j) for s_ in succ[j])
    return found


def test_hazard_scan_finds_planted_hazards():
    """The scanner itself: a VALU write just before an inline MFMA, one two
    wait states away, a result read through a taken branch, and a distant read."""
    asm = """
_Zfoo:
	v_mov_b32_e32 v5, v1
	;;#ASMSTART
	v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[4:7], v[16:31]
	;;#ASMEND
	s_cbranch_scc1 .LBB0_2
	s_nop 7
	s_nop 7
	s_nop 7
	v_add_f32_e32 v40, v16, v40
.LBB0_2:
	v_add_f32_e32 v41, v17, v41
	v_mov_b32_e32 v2, v9
	s_nop 1
	;;#ASMSTART
	v_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], v[4:7], 0
	;;#ASMEND
	s_endpgm
.Lfunc_end0:
"""
    found = _hazards(_functions(asm)["_Zfoo"])
    assert any("v_mov_b32_e32 v5" in f and "(0 wait states)" in f for f in found), found
    assert any("v_add_f32_e32 v41, v17" in f and "(1 wait states)" in f for f in found), found
    assert not any("v40" in f or "v_mov_b32_e32 v2" in f for f in found), found
    # a wave-uniform if around the MFMA and around its readers: the path that
    # issues the MFMA and skips the delay cannot happen, unless the tested
    # value is rewritten in between
    tmpl = """
_Zbar:
	s_and_b64 vcc, exec, s[2:3]
	s_cbranch_vccnz .LBB1_1
	;;#ASMSTART
	v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[4:7], v[16:31]
	;;#ASMEND
.LBB1_1:
	{mid}
	s_and_b64 vcc, exec, s[2:3]
	s_cbranch_vccnz .LBB1_2
	s_nop 7
	s_nop 7
	s_nop 7
	v_add_f32_e32 v40, v16, v40
.LBB1_2:
	v_mov_b32_e32 v16, 0
	s_endpgm
.Lfunc_end1:
"""
    assert _hazards(_functions(tmpl.format(mid="s_nop 0"))["_Zbar"]) == []
    found = _hazards(_functions(tmpl.format(mid="s_mov_b64 s[2:3], -1"))["_Zbar"])
    assert any("v_mov_b32_e32 v16, 0" in f for f in found), found


def test_inline_mfma_hazards_resolved(reports):
    checked, bad = 0, []
    for src, kernels in reports.items():
        for name, lines in _functions(kernels["__asm__"]).items():
            if not any("v_mfma" in l for l in lines) or not any("ASMSTART" in l for l in lines):
                continue
            checked += 1
            bad += [f"{name[-48:]}: {h}" for h in _hazards(lines)]
    assert checked >= 16
    assert not bad, "\n".join(bad[:20])
