"""Checks on the gfx950 code the library compiles to (host-side: hipcc cross-compiles, no GPU).

The direct-to-LDS loads write M0 (the instruction's LDS base) without saving it, which is sound
only while no compiler-generated instruction in the library reads or writes M0.  This test
compiles the library to assembly and fails if any instruction outside the inline-assembly loads
names M0, if an inline-assembly block that writes SCC sits where the compiler keeps SCC live
across it, if the kernels spill registers to scratch memory, and if the LDS the planner reports
for a tile and operand layout differs from what the compiled kernel declares.
"""
import os
import re
import shutil

import pytest

from dense_tiled_gemm_f16_amd import build


@pytest.fixture(scope="module", params=["product", "measurement"])
def asm_text(request, tmp_path_factory):
    """The product library's sources, then the measurement library's (its load-latency probe writes
    M0 the same way)."""
    if shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not available")
    sources = build.SOURCES if request.param == "product" else build.MEASURE_SOURCES
    outs = build.emit_asm(str(tmp_path_factory.mktemp("asm")), sources=sources)
    return "\n".join(open(o).read() for o in outs)


def test_m0_is_used_only_by_the_direct_to_lds_loads(asm_text):
    outside = re.sub(r";;#ASMSTART.*?;;#ASMEND", "", asm_text, flags=re.S)
    uses = [l for l in outside.splitlines() if re.search(r"\bm0\b", l) and not l.lstrip().startswith(";")]
    assert uses == [], uses[:5]
    inside = re.findall(r";;#ASMSTART(.*?);;#ASMEND", asm_text, flags=re.S)
    assert any("global_load_lds_dwordx4" in b and "m0" in b for b in inside)


# Scalar instructions that write SCC, and those that read it (gfx9).
_SCC_WRITERS = re.compile(r"^\s*(s_cmp\w*|s_cmpk\w*|s_bitcmp\w*|s_add_u32|s_add_i32|s_addc_u32|s_addk_i32|s_sub_u32|"
                          r"s_sub_i32|s_subb_u32|s_and_b\d+|s_or_b\d+|s_xor_b\d+|s_andn2_b\d+|s_orn2_b\d+|s_nand_b\d+|"
                          r"s_nor_b\d+|s_xnor_b\d+|s_not_b\d+|s_lshl\w*|s_lshr\w*|s_ashr\w*|s_min_\w*|s_max_\w*|s_bfe\w*|"
                          r"s_abs\w*|s_absdiff\w*|s_bcnt\w*|s_quadmask\w*|s_wqm\w*)\b")
_SCC_READERS = re.compile(r"^\s*(s_cselect\w*|s_cbranch_scc\d|s_addc_u32|s_subb_u32|s_cmov\w*)\b")


def test_inline_asm_does_not_break_a_live_scc(asm_text):
    """The direct-to-LDS loads form M0 with s_add_u32, which writes SCC.  If the compiler kept a
    carry or a comparison in SCC across such a block -- an address add split around it -- the
    value read after it would be the block's, and a 64-bit address would come out 2^32 bytes off.
    No SCC reader may follow a block that writes SCC before SCC is written again."""
    lines = asm_text.splitlines()
    bad = []
    k = 0
    while k < len(lines):
        if ";;#ASMSTART" in lines[k]:
            end = k
            while ";;#ASMEND" not in lines[end]:
                end += 1
            if any(_SCC_WRITERS.match(l) for l in lines[k + 1:end]):
                for m in range(end + 1, len(lines)):
                    l = lines[m]
                    if ";;#ASMSTART" in l or re.match(r"^\s*s_endpgm", l) or re.match(r"^\S.*:", l):
                        break
                    if _SCC_READERS.match(l):
                        bad.append(l.strip())
                        break
                    if _SCC_WRITERS.match(l):
                        break
            k = end
        k += 1
    assert bad == [], bad[:5]


def test_kernels_do_not_spill(asm_text):
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm_text) + re.findall(r"\.sgpr_spill_count:\s+(\d+)", asm_text)
    assert spills and all(int(x) == 0 for x in spills), spills



def _kernel_lds(asm_text):
    """{(bm, bn, bk, ks, ta, tb): LDS bytes} of every product GEMM kernel, from the code-object metadata
    (each kernel's .group_segment_fixed_size precedes its .name)."""
    out, size = {}, None
    for line in asm_text.splitlines():
        m = re.match(r"\s+\.group_segment_fixed_size:\s+(\d+)", line)
        if m:
            size = int(m.group(1))
            continue
        m = re.match(r"\s+\.name:\s+\S*gemm_f16_f32_kernel\S*TileILi(\d+)ELi(\d+)ELi(\d+)ELi\d+ELi\d+ELi\d+"
                     r"ELi\d+ELi(\d+)ELb([01])ELb([01])E", line)
        if m:
            out[tuple(int(x) for x in m.groups())] = size
    return out


def test_planned_lds_matches_the_compiled_kernels(asm_text):
    if "gemm_f16_f32_kernel" not in asm_text:
        pytest.skip("measurement sources")
    from dense_tiled_gemm_f16_amd import _abi as g
    declared = _kernel_lds(asm_text)
    assert len(declared) >= 20, sorted(declared)
    n = 4096
    for tile in range(1, 6):
        for ta in (0, 1):
            for tb in (0, 1):
                rc, p = g.gemm_f16_f32_plan_tt(ta, tb, n, n, n, 256, n, 256, n, 256, n, {"tile": tile})
                assert rc == 0
                key = (p["bm"], p["bn"], p["bk"], 4 if tile == 5 else 1, ta, tb)
                assert declared[key] == p["lds_bytes"], (tile, ta, tb, declared[key], p["lds_bytes"])
