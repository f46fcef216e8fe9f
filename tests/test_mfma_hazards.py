"""Static check of the device assembly for reads of a matrix product's result too soon after it.

Several kernels issue their MFMA products as inline asm, so that the compiler keeps them in a
hand-chosen order. The compiler does not know an inline-asm instruction's latency, so it puts
no wait states between such a product and a later instruction that reads its destination
registers; the kernels pad those reads themselves (s_nop after the last product of a tile). A
register copy that the compiler inserts on its own (where two control paths join, say) can
land between a product and that padding and read an accumulator before the product has
written it: the result is silently wrong. This test compiles each source that holds inline-asm
products to gfx950 assembly and checks that no instruction reads a product's destination
within 19 wait states of an inline-asm product (the requirement of a 16-pass XDL product on
CDNA3/CDNA4, the longest of the products used here). A product that reads the same registers
as its accumulator input is exempt: the hardware chains dependent products itself. The other
direction is checked too: a vector-ALU instruction (register copies included) that writes a
register an inline-asm product reads as an operand needs 2 wait states before that product.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_flash_amd", "csrc")
WAIT_STATES = 19
VALU_TO_MFMA_WAIT_STATES = 2

_REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _operands(ins):
    parts = ins.split(None, 1)
    return parts[1].split(",") if len(parts) > 1 else []


def find_hazards(asm_lines, wait_states=WAIT_STATES):
    """(line of product, line of early reader, wait states between) for each hazard found.

    Only products written as inline asm are checked (the compiler pads its own). The scan of a
    product stops at a branch, a label, a barrier or the end of the program, so a read on the
    other side of one is not seen (a barrier stalls for far longer than any product)."""
    found = []
    for i, line in enumerate(asm_lines):
        ins = line.strip()
        if not ins.startswith("v_mfma") or i == 0 or "ASMSTART" not in asm_lines[i - 1]:
            continue
        dst = _regs(_operands(ins)[0])
        dist = 0
        for k in range(i + 1, len(asm_lines)):
            u = asm_lines[k].strip()
            if u.startswith((".LBB", ".Lfunc_end", "s_barrier", "s_endpgm", "s_cbranch", "s_branch")):
                break
            if not u or u.startswith((";", ".")):
                continue
            if u.startswith("s_nop"):
                dist += int(u.split()[1]) + 1
            else:
                op, ops = u.split()[0], _operands(u)
                if op.startswith("v_mfma"):
                    srcs = _regs(",".join(ops[1:3]))   # srcC chaining is interlocked
                elif op.startswith(("ds_write", "buffer_store", "global_store", "flat_store")):
                    srcs = _regs(",".join(ops))
                else:
                    srcs = _regs(",".join(ops[1:]))
                if srcs & dst:
                    found.append((i + 1, k + 1, dist))
                    break
                if op.startswith("v_mfma") and _regs(ops[0]) & dst:
                    break   # a later product owns these registers now
                dist += 1
            if dist >= wait_states:
                break
    return found


def find_operand_hazards(asm_lines, wait_states=VALU_TO_MFMA_WAIT_STATES):
    """(line of product, line of the writer, wait states between) for each vector-ALU write of
    an inline-asm product's operand (A, B or accumulator input) too close before it. The scan
    back stops at a label, a branch or a barrier."""
    found = []
    for i, line in enumerate(asm_lines):
        ins = line.strip()
        if not ins.startswith("v_mfma") or i == 0 or "ASMSTART" not in asm_lines[i - 1]:
            continue
        srcs = _regs(",".join(_operands(ins)[1:4]))
        dist = 0
        for k in range(i - 1, -1, -1):
            u = asm_lines[k].strip()
            if u.startswith((".LBB", "s_barrier", "s_cbranch", "s_branch")) or re.match(r"^_Z\S+:", u):
                break
            if not u or u.startswith((";", ".")):
                continue
            if u.startswith("s_nop"):
                dist += int(u.split()[1]) + 1
            else:
                op, ops = u.split()[0], _operands(u)
                if op.startswith("v_") and not op.startswith("v_mfma") and ops and _regs(ops[0]) & srcs:
                    found.append((i + 1, k + 1, dist))
                    break
                dist += 1
            if dist >= wait_states:
                break
    return found


def test_checker_flags_early_reads():
    # the checker itself: an early copy is flagged, padded and chained reads are not
    early = ["\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
             "\t;;#ASMEND", "\tv_add_u32_e32 v9, 1, v9", "\tv_accvgpr_mov_b32 a20, a3"]
    assert find_hazards(early) == [(2, 5, 1)]
    padded = early[:3] + ["\ts_nop 7", "\ts_nop 7", "\ts_nop 3"] + early[4:]
    assert find_hazards(padded) == []
    chained = early[:3] + ["\tv_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[4:7], a[0:15]"]
    assert find_hazards(chained) == []
    other = early[:3] + ["\tv_accvgpr_read_b32 v2, a16"]
    assert find_hazards(other) == []
    compiler = ["\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
                "\tv_accvgpr_read_b32 v2, a0"]
    assert find_hazards(compiler) == []

    # a copy into the accumulator right before the product, then the same with padding
    copy = ["\tv_accvgpr_mov_b32 a3, a19", "\ts_waitcnt lgkmcnt(0)"] + early[:3]
    assert find_operand_hazards(copy) == [(4, 1, 1)]
    assert find_operand_hazards(copy[:1] + ["\ts_nop 1"] + copy[1:]) == []
    operand = ["\tv_cvt_pk_bf16_f32 v5, v8, v9"] + early[:3]
    assert find_operand_hazards(operand) == [(3, 1, 0)]
    unrelated = ["\tv_cvt_pk_bf16_f32 v12, v8, v9"] + early[:3]
    assert find_operand_hazards(unrelated) == []


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    from exact_tiled_attention_flash_amd import build as b
    tmp = tmp_path_factory.mktemp("asm")
    srcs = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip"):
            with open(os.path.join(CSRC, f)) as fh:
                text = fh.read()
            if "v_mfma" in text or "fa_fwd_parts.h" in text:
                srcs.append(f)

    def compile_one(f):
        out = os.path.join(tmp, f + ".s")
        subprocess.run([hipcc, f"--offload-arch={b.ARCH}", *b.COMMON, *b.DEVICE_FLAGS,
                        *b.EXTRA.get(f, []), "--cuda-device-only", "-S",
                        os.path.join(CSRC, f), "-o", out],
                       cwd=CSRC, capture_output=True, text=True, check=True)
        with open(out) as fh:
            return f, fh.read().splitlines()

    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        return dict(ex.map(compile_one, srcs))


def test_inline_asm_products_are_padded(assembly):
    assert "fa_fwd_bf16.hip" in assembly
    report, total = [], 0
    for f, lines in assembly.items():
        n_asm = sum(1 for i, l in enumerate(lines)
                    if l.strip().startswith("v_mfma") and i and "ASMSTART" in lines[i - 1])
        hz, ow = find_hazards(lines), find_operand_hazards(lines)
        total += len(hz) + len(ow)
        report.append(f"{f}: {n_asm} inline-asm products, {len(hz)} early reads, "
                      f"{len(ow)} late operand writes")
        for p, r, d in hz[:5]:
            report.append(f"  product at line {p}: read at line {r} after {d} wait states: "
                          f"{lines[r - 1].strip()}")
        for p, w, d in ow[:5]:
            report.append(f"  product at line {p}: operand written at line {w}, {d} wait states "
                          f"before: {lines[w - 1].strip()}")
    print("\n".join(report))
    assert total == 0, "\n".join(report)
