"""Wait states around the inline-assembly MFMAs (CPU only).

The compiler pads its own MFMAs with the wait states the matrix pipe needs, but treats an
inline-assembly statement as opaque. The kernels issue some 8-pass XDL MFMAs as inline
assembly, so that the VALU reads their results straight from VGPRs. These tests compile
every device source that does so to gfx950 assembly with the library's own flags, and check
each such MFMA against the compiler's own wait-state model for 8-pass XDL operations. The
thresholds are the ones it uses: its gfx950 code never has fewer between its own MFMAs and
their neighbours. Counting: one wait state per instruction and N+1 for ``s_nop N``, as the
compiler counts; after the MFMA, each further MFMA counts as 4 (one pass): it cannot enter
the matrix pipe before the one ahead of it has held the pipe for a pass. That is a loose
lower bound: at the chip's dense peak an 8-pass MFMA holds the pipe for 32 cycles. The rules
are:

* a VALU write of a source register needs 2 wait states before the MFMA;
* a separate accumulator input (srcC, when it is not the result register) may be written
  again, by a VALU op or a load's return, only 8 wait states after the issue;
* the result may be read or written by anything but a chained MFMA on the same accumulator
  (exact overlap of srcC and result) only 12 wait states after the issue.

A label or branch inside one of these windows counts as a violation: the check does not
follow control flow.

The same assembly (plus the backward's) also carries the kernels' resource metadata: the
kernels whose speed rests on their register and LDS budgets must compile with no VGPR spills
and within the LDS that their residency assumes.
"""
import glob
import os
import re
import subprocess

import pytest

from jl_feature_projected_amd import build as B

RAW_BEFORE = 2
SRCC_WAR = 8
RESULT_AFTER = 12
MFMA_BEHIND = 4


def _regs(tok: str) -> set:
    tok = tok.strip()
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


class Inst:
    __slots__ = ("op", "ops", "asm", "line", "text")

    def __init__(self, op, ops, asm, line, text):
        self.op, self.ops, self.asm, self.line, self.text = op, ops, asm, line, text

    @property
    def boundary(self) -> bool:
        return self.op == "LABEL" or self.op.startswith(("s_branch", "s_cbranch", "s_setpc",
                                                         "s_endpgm"))

    @property
    def is_mfma(self) -> bool:
        return self.op.startswith("v_mfma")

    def wait_states(self) -> int:
        return int(self.ops[0], 0) + 1 if self.op == "s_nop" else 1

    def defs(self) -> set:
        if not self.ops or self.op.startswith(("ds_write", "ds_store", "buffer_store",
                                               "global_store", "flat_store", "scratch_store")):
            return set()
        if self.op.startswith("buffer_load") and self.ops[-1].split()[-1] == "lds":
            return set()  # the LDS-direct form writes no VGPR
        if self.op.startswith(("v_", "ds_", "buffer_", "global_", "flat_", "scratch_")):
            return _regs(self.ops[0])
        return set()

    def uses(self) -> set:
        d = self.defs()
        toks = self.ops[1:] if d else self.ops
        out = set()
        for t in toks:
            for part in t.split():
                out |= _regs(part)
        return out


def parse(text: str):
    """Instruction stream per function: (name, [Inst])."""
    funcs, cur, name, in_asm = [], None, None, False
    for n, raw in enumerate(text.split("\n"), 1):
        s = raw.strip()
        m = re.match(r"^(_Z\S+):", s)
        if m:
            name, cur = m.group(1), []
            funcs.append((name, cur))
            continue
        if cur is None:
            continue
        if ";;#ASMSTART" in s:
            in_asm = True
            continue
        if ";;#ASMEND" in s:
            in_asm = False
            continue
        if re.match(r"^\.LBB\d+_\d+:", s):
            cur.append(Inst("LABEL", [], in_asm, n, s))
            continue
        s = s.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        cur.append(Inst(parts[0], ops, in_asm, n, s))
    return funcs


def check(text: str) -> list:
    """Violations of the three rules at every inline-assembly MFMA of ``text``."""
    bad = []
    for name, insts in parse(text):
        for k, mf in enumerate(insts):
            if not (mf.asm and mf.is_mfma):
                continue
            dst = _regs(mf.ops[0])
            srcab = _regs(mf.ops[1]) | _regs(mf.ops[2])
            srcc = _regs(mf.ops[3])
            chained = srcc == dst

            def report(rule, other):
                bad.append(f"{name[:60]}: line {mf.line} '{mf.text}' / line {other.line} "
                           f"'{other.text}': {rule}")

            # before: VALU writes of a source; MFMA results used as a source
            ws = 0
            for j in range(k - 1, -1, -1):
                o = insts[j]
                if ws >= RESULT_AFTER:
                    break
                if o.boundary:
                    if ws < RAW_BEFORE:
                        report("control flow right before the MFMA", o)
                    break
                w = o.defs()
                if o.is_mfma:
                    if w & (srcab | srcc) and not (chained and w == dst and _regs(o.ops[3]) == w):
                        report(f"MFMA result used {ws} wait states later", o)
                elif ws < RAW_BEFORE and w & (srcab | srcc):
                    report(f"VALU write {ws} wait states before the MFMA", o)
                ws += o.wait_states()
            # after: srcC rewritten, result touched
            ws = 0
            for j in range(k + 1, len(insts)):
                o = insts[j]
                if ws >= max(RESULT_AFTER, SRCC_WAR):
                    break
                if o.boundary:
                    report(f"control flow {ws} wait states after the MFMA", o)
                    break
                if o.is_mfma and _regs(o.ops[3]) == dst and _regs(o.ops[0]) == dst:
                    # a chained MFMA continues the accumulation; it is checked in turn, and
                    # the original srcC stays covered by the rule below
                    if not chained and ws < SRCC_WAR and (srcc - dst) & o.defs():
                        report(f"srcC rewritten {ws} wait states after the MFMA", o)
                    break
                touched = o.defs() | o.uses()
                if ws < RESULT_AFTER and touched & dst:
                    report(f"result touched {ws} wait states after the MFMA", o)
                if not chained and ws < SRCC_WAR and o.defs() & (srcc - dst):
                    report(f"srcC rewritten {ws} wait states after the MFMA", o)
                ws += MFMA_BEHIND if o.is_mfma else o.wait_states()
    return bad


def _sources_with_asm_mfmas() -> list:
    helpers = set()
    for hdr in glob.glob(os.path.join(B.CSRC, "*.h")):
        txt = open(hdr).read()
        for m in re.finditer(r"__forceinline__\s+\S+\s+(\w+)\([^)]*\)\s*\{[^}]*asm[^}]*v_mfma", txt):
            helpers.add(m.group(1))
    out = []
    for src in sorted(glob.glob(os.path.join(B.CSRC, "*.hip"))):
        txt = open(src).read()
        if re.search(r"asm[^;]*v_mfma", txt) or any(re.search(rf"\b{h}\(", txt) for h in helpers):
            out.append(src)
    return out


def test_the_checker_sees_planted_hazards():
    # A hand-written stream with one violation of each rule, then the same stream padded.
    bad = """
_Zk:
v_mov_b32 v5, v9
;;#ASMSTART
v_mfma_f32_32x32x16_f16 v[16:31], v[0:3], v[4:7], v[32:47]
;;#ASMEND
ds_read_b128 v[32:35], v1
v_exp_f32_e32 v40, v16
"""
    found = check(bad)
    assert any("VALU write 0 wait states" in f for f in found), found
    assert any("srcC rewritten 0 wait states" in f for f in found), found
    assert any("result touched 1 wait states" in f for f in found), found
    good = """
_Zk:
v_mov_b32 v5, v9
;;#ASMSTART
s_nop 1
v_mfma_f32_32x32x16_f16 v[16:31], v[0:3], v[4:7], v[32:47]
s_nop 7
;;#ASMEND
ds_read_b128 v[32:35], v1
s_nop 2
v_exp_f32_e32 v40, v16
"""
    assert check(good) == []
    # a chain on one accumulator needs no wait between its links
    chain = """
_Zk:
s_nop 1
;;#ASMSTART
s_nop 1
v_mfma_f32_32x32x16_f16 v[16:31], v[0:3], v[4:7], v[16:31]
;;#ASMEND
;;#ASMSTART
s_nop 1
v_mfma_f32_32x32x16_f16 v[16:31], v[8:11], v[12:15], v[16:31]
;;#ASMEND
s_nop 15
v_exp_f32_e32 v40, v16
"""
    assert check(chain) == []


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """gfx950 assembly of the sources with inline MFMAs and of the backward, by file name."""
    if not os.path.exists(B.hipcc()):
        pytest.skip("hipcc is not installed")
    out_dir = tmp_path_factory.mktemp("asm")
    srcs = sorted(set(_sources_with_asm_mfmas()) | {os.path.join(B.CSRC, "spa_bwd.hip")})
    texts = {}
    for src in srcs:
        out = str(out_dir / (os.path.basename(src) + ".s"))
        subprocess.run([B.hipcc(), *B.compile_flags(), "--cuda-device-only", "-S", src, "-o", out],
                       check=True, capture_output=True, text=True)
        texts[os.path.basename(src)] = open(out).read()
    return texts


def test_inline_asm_mfmas_keep_their_wait_states(device_asm):
    srcs = _sources_with_asm_mfmas()
    assert srcs, "no device source issues an inline-assembly MFMA"
    problems = []
    for src in srcs:
        text = device_asm[os.path.basename(src)]
        assert re.search(r";;#ASMSTART\s*\n\s*(s_nop \d+\s*\n\s*)?v_mfma", text), src
        problems += [f"{os.path.basename(src)}: {p}" for p in check(text)]
    assert not problems, "\n".join(problems[:40])


def _kernel_resources(text: str) -> dict:
    """Per kernel symbol: vgpr_count, vgpr_spill_count, group_segment_fixed_size (LDS)."""
    out = {}
    for blk in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        field = lambda f: int(re.search(rf"\.{f}:\s+(\d+)", blk).group(1))
        out[name] = {"vgpr": field("vgpr_count"), "vgpr_spill": field("vgpr_spill_count"),
                     "lds": field("group_segment_fixed_size")}
    return out


# The kernels whose speed rests on their register and LDS budgets: the one-wave attention
# variant (every register of the SIMD, no spill code in or around its ring) and the fused
# key-major backward kernel (two workgroups per CU: at most 256 registers, half the LDS).
HOT = [
    ("spa_attn_bf16.hip", r"attn_bf16_kernelILi(16|32)ELi128ELb[01]ELi2E", 163840),
    ("spa_bwd.hip", r"bwd_kv_kernelILi(16|32)ELi128ELb[01]ELb1E", 81920),
]


@pytest.mark.parametrize("src,pattern,lds_max", HOT, ids=["attention-one-wave", "bwd-key-major-fused"])
def test_hot_kernels_keep_their_budgets(device_asm, src, pattern, lds_max):
    res = {k: v for k, v in _kernel_resources(device_asm[src]).items() if re.search(pattern, k)}
    assert len(res) == 4, sorted(res)
    for name, r in res.items():
        assert r["vgpr_spill"] == 0, (name, r)
        assert r["lds"] <= lds_max, (name, r)
