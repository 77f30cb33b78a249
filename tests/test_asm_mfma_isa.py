"""ISA checks on the kernels that issue their MFMAs from inline asm.

The 16x16x32 main loop (csrc/gemm_core.h) issues v_mfma_f32_16x16x32 from
inline asm so its accumulators stay in AGPRs. The compiler inserts no hazard
waits around asm, so the loop relies on properties of the generated code
that these tests check on the gfx950 assembly of every kernel built on it:

* no VALU instruction writes an accumulator (AGPR) at all: each accumulator
  starts with an MFMA whose addend is the constant 0;
* every other instruction that touches an AGPR comes after an s_nop wait that
  follows the last MFMA before it (the explicit wait at the end of the loop);
* no VALU instruction writes an MFMA operand within 6 wait states before it;
* an s_waitcnt lgkmcnt covers every LDS read before an MFMA reads its result
  (the compiler places these from the asm's register operands).

The checks run on the text of the assembly in program order; inside the
k-loop every region ends with lgkmcnt(0) before its barrier, so nothing is
pending across the loop's back edge.
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from post_weight_quantization_26_amd import build_lib

KERNELS = {
    "gemm.hip": [r"search_gemm_bf16_kernel", r"search_gemm_f16_kernel",
                 r"search_gemm_bf16_split_kernel", r"search_gemm_f16_split_kernel"],
    "gram.hip": [r"gram_partial_kernel", r"gram_search_kernel"],
    "w4a16.hip": [r"w4a16_gemm_kernelILb0", r"w4a16_gemm_kernelILb1", r"w4a16_gemm_q_kernelILb0",
                  r"w4a16_gemm_q_kernelILb1"],
    "fused.hip": [r"search_fused_kernelILb0", r"search_fused_kernelILb1"],
}


def _hipcc():
    try:
        return build_lib.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("isa")

    def compile_one(src):
        dst = str(out / (src + ".s"))
        cmd = [cc, *build_lib.COMMON, "--cuda-device-only", "-S",
               os.path.join(build_lib.CSRC, src), "-o", dst]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return src, open(dst).read()

    with cf.ThreadPoolExecutor(len(KERNELS)) as ex:
        return dict(ex.map(compile_one, KERNELS))


def _kernel_body(asm, name):
    m = re.search(r"^(_Z\S*" + name + r"\S*):[ \t]*(;.*)?$", asm, re.M)
    assert m, f"kernel {name} not found in the assembly"
    # the whole function: a kernel may end early on some paths (padding blocks)
    fe = asm.find(".Lfunc_end", m.end())
    end = fe if fe >= 0 else asm.index("s_endpgm", m.end())
    lines = asm[m.end():end].split("\n")
    return [ln.strip() for ln in lines
            if ln.strip() and not ln.strip().startswith((";", ".", "#"))]


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)\b", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _operands(ins):
    parts = ins.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


def _mfma_regs(ins):
    ops = _operands(ins)
    dst = _regs(ops[0])
    src = set().union(*(_regs(t.split()[0]) for t in ops[1:4]))
    return dst, src


def _cases():
    return [(src, k) for src, names in KERNELS.items() for k in names]


@pytest.mark.parametrize("src,kernel", _cases())
def test_asm_mfma_kernel_isa(assembly, src, kernel):
    ins = _kernel_body(assembly[src], kernel)
    mfma = [i for i, s in enumerate(ins) if s.startswith("v_mfma_f32_16x16x32")]
    assert len(mfma) >= 128, f"{kernel}: expected the 16x16x32 loop, found {len(mfma)} MFMAs"
    nops = [i for i, s in enumerate(ins) if re.match(r"s_nop (\d+)", s) and int(s.split()[1]) >= 7]

    # 1. no VALU write of an AGPR anywhere
    writes = [s for s in ins if s.startswith(("v_accvgpr_write", "v_accvgpr_mov"))]
    assert not writes, f"{kernel}: VALU writes to accumulators: {writes[:3]}"

    # 2. every non-MFMA use of an AGPR follows a wait placed after the last MFMA
    for i, s in enumerate(ins):
        if s.startswith("v_mfma") or not any(r[0] == "a" for t in _operands(s) for r in _regs(t)):
            continue
        last = max((m for m in mfma if m < i), default=-1)
        assert any(last < n < i for n in nops), f"{kernel}: AGPR use without a wait: {s}"

    # 3. VALU writes of MFMA operands at least 6 wait states before the MFMA
    for k in mfma:
        dst, src_regs = _mfma_regs(ins[k])
        states = 0
        for b in range(1, 40):
            p = ins[k - b]
            m = re.match(r"s_nop (\d+)", p)
            states += int(m.group(1)) + 1 if m else 1
            if states > 6:
                break
            if p.startswith("v_") and not p.startswith(("v_mfma", "v_readfirstlane")):
                ops = _operands(p)
                if ops:
                    assert not (_regs(ops[0]) & (src_regs | dst)), \
                        f"{kernel}: VALU write {states} states before MFMA: {p} -> {ins[k]}"

    # 4. LDS read results waited for before an MFMA reads them. lgkmcnt
    # counts every LDS and scalar-memory operation in issue order (a loop
    # that forms an operand in registers stores it to LDS among the reads),
    # so all of them enter the queue; only reads carry registers.
    pending = []
    for s in ins:
        if s.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if 0 < n < len(pending) else ([] if n == 0 else pending)
            continue
        if s.startswith("ds_read"):
            pending.append(_regs(_operands(s)[0]))
        elif s.startswith(("ds_write", "s_load", "s_buffer_load")):
            pending.append(set())
        elif s.startswith("v_mfma"):
            _, src_regs = _mfma_regs(s)
            assert not any(p & src_regs for p in pending), f"{kernel}: MFMA reads an LDS result in flight: {s}"
