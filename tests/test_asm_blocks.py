"""The generated inline-assembly blocks of the MFMA attention kernel: the
committed include matches its generator, and a replay of each block finds no
LDS read consumed before it landed, no ring slot overwritten too early and
no scalar load left unwaited at the end of a block."""
import importlib.util
import subprocess

import pytest
import sys
from pathlib import Path

CSRC = Path(__file__).resolve().parents[1] / "paged_mla_latent_write_amd" / "csrc"


def _load(name):
    spec = importlib.util.spec_from_file_location(name, CSRC / f"{name}.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_include_matches_generator():
    out = subprocess.run([sys.executable, str(CSRC / "gen_attn_mfma_asm.py")], capture_output=True, text=True,
                         check=True).stdout
    assert out == (CSRC / "attn_mfma_asm.inc").read_text()


def test_fp8_include_matches_generator():
    out = subprocess.run([sys.executable, str(CSRC / "gen_attn_mfma_asm.py"), "--fp8"], capture_output=True,
                         text=True, check=True).stdout
    assert out == (CSRC / "attn_mfma_fp8_asm.inc").read_text()


def test_fp8_blocks_wait_for_their_lds_reads():
    n, problems = _load("check_attn_mfma_asm").check((CSRC / "attn_mfma_fp8_asm.inc").read_text())
    assert n == 15 and not problems, problems[:5]


def test_checker_catches_a_conversion_before_its_codes_landed():
    # plant a mistake: drop the waits of one fp8 block's scores half (the
    # conversions then read code registers whose LDS reads are in flight)
    text = (CSRC / "attn_mfma_fp8_asm.inc").read_text()
    start = text.index("void fp8_step_tail_f0_m0(")
    cut = text.index("v_mfma_f32_32x32x16_bf16 v[208:223], v[232:235], v[86:89]", start)
    planted = text[:start] + text[start:cut].replace("s_waitcnt lgkmcnt(", "s_nop 0 // (") + text[cut:]
    n, problems = _load("check_attn_mfma_asm").check(planted)
    assert any("VALU use of a register whose LDS read has not landed" in p for p in problems)


def test_checker_catches_a_write_source_overwritten_too_early():
    # plant a mistake: a conversion overwrites the values the previous
    # half's LDS write may still be reading
    text = (CSRC / "attn_mfma_fp8_asm.inc").read_text()
    start = text.index("void fp8_step_tail_f0_m0(")
    first = text.index("ds_write_b128 v206", start)
    nxt = text.index("v_cvt_scalef32_pk_bf16_fp8", first)
    wait = text.rindex("s_waitcnt lgkmcnt(", first, nxt)
    planted = text[:wait] + "s_nop 0 // (" + text[wait + len("s_waitcnt lgkmcnt("):]
    n, problems = _load("check_attn_mfma_asm").check(planted)
    assert any("LDS write still reads" in p for p in problems)


def test_blocks_wait_for_their_lds_reads():
    n, problems = _load("check_attn_mfma_asm").check((CSRC / "attn_mfma_asm.inc").read_text())
    assert n > 10 and not problems, problems[:5]


def test_checker_catches_a_ring_slot_reused_too_early():
    # plant a mistake: drop every lgkmcnt wait from one block
    text = (CSRC / "attn_mfma_asm.inc").read_text()
    start = text.index("void tile_step_tail_d1_f0_m0(")
    end = text.index("\n}\n", start)
    planted = text[:start] + text[start:end].replace("s_waitcnt lgkmcnt(", "s_nop 0 // (") + text[end:]
    n, problems = _load("check_attn_mfma_asm").check(planted)
    assert problems


def test_checker_catches_an_unwaited_scalar_load():
    # plant a mistake: drop the waits that follow the block-table read
    text = (CSRC / "attn_mfma_asm.inc").read_text()
    start = text.index("void tile_hot_loop(")
    end = text.index("\n}\n", start)
    body = text[start:end]
    assert "s_load_dword" in body
    planted = text[:start] + body.replace("s_waitcnt lgkmcnt(0)", "s_waitcnt lgkmcnt(1)") + text[end:]
    n, problems = _load("check_attn_mfma_asm").check(planted)
    assert any("scalar load" in p for p in problems)


def test_checker_follows_reads_across_the_loop_back_edge():
    # plant a mistake: the hot loop's first wait no longer covers the K
    # fragments its previous pass read (only a two-pass replay sees them)
    text = (CSRC / "attn_mfma_asm.inc").read_text()
    start = text.index("void tile_hot_loop(")
    end = text.index("\n}\n", start)
    body = text[start:end]
    top = body.index('"1:\\n"')
    w = body.index("s_waitcnt lgkmcnt(", top)
    planted = text[:start] + body[:w] + "s_waitcnt lgkmcnt(9)" + body[body.index(")", w) + 1:] + text[end:]
    n, problems = _load("check_attn_mfma_asm").check(planted)
    assert any("tile_hot_loop: MFMA before its LDS read landed" in p for p in problems)


def _compiler_registers(src):
    """Highest VGPR index and number of AGPR references in the compiler's own
    code (outside the inline-assembly blocks) of one kernel source."""
    import re
    import shutil
    import tempfile

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    with tempfile.TemporaryDirectory() as d:
        out = Path(d) / "k.s"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-I", str(CSRC), "-I", str(CSRC.parents[1] / "include"),
                        "-x", "hip", "--cuda-device-only", "-S", str(CSRC / src), "-o", str(out)],
                       check=True, capture_output=True)
        text = out.read_text()
    top, agprs, in_asm = -1, 0, False
    for ln in text.splitlines():
        if ";;#ASMSTART" in ln:
            in_asm = True
        elif ";;#ASMEND" in ln:
            in_asm = False
        elif not in_asm and ln.startswith("\t") and not ln.startswith("\t."):
            for m in re.finditer(r"\bv(\d+)\b|v\[(\d+):(\d+)\]", ln):
                top = max(top, int(m.group(1) or m.group(3)))
            agprs += len(re.findall(r"\ba(\d+)\b|a\[\d+:\d+\]", ln))
    return top, agprs


@pytest.mark.parametrize("src", ["attn_mfma.hip", "attn_mfma_fp8.hip"])
def test_compiler_code_leaves_reserved_registers_alone(src):
    """The queries, scores, ring and accumulators live in registers the blocks
    own from one block to the next.  amdgpu_num_vgpr only steers the compiler
    (under pressure it goes past it), so the compiled kernel is checked: its
    own code may use the registers of the previous tile's P (each block that
    reads them writes them first) but nothing from the queries up."""
    import shutil

    if not (shutil.which("hipcc") or Path("/opt/rocm/bin/hipcc").exists()):
        pytest.skip("hipcc not available")
    gen = _load("gen_attn_mfma_asm")
    top, agprs = _compiler_registers(src)
    assert top < gen.Q_BASE, f"{src}: compiler code uses v{top} (queries start at v{gen.Q_BASE})"
    assert agprs == 0, f"{src}: compiler code references accumulator registers"


def test_fp8_matrix_core_kernel_keeps_its_registers():
    """The fp8-MFMA attention kernel holds 16 accumulator tiles (all 256
    accumulation registers) and its score accumulators in VGPRs: its step
    loop must run without spilling to scratch, and its score MFMAs must
    accumulate in VGPRs (not in the accumulation registers the values use)."""
    import re
    import shutil
    import tempfile

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = Path(d) / "k.s"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-I", str(CSRC), "-I", str(CSRC.parents[1] / "include"),
                        "-x", "hip", "--cuda-device-only", "-S", str(CSRC / "attn_f8mfma.hip"), "-o", str(out)],
                       check=True, capture_output=True)
        text = out.read_text()
    # no scratch traffic inside the step loop (the compiler marks the blocks
    # of nested loops "Depth=2"); a few spills per segment are harmless
    depth, in_loop_scratch = 0, 0
    for ln in text.splitlines():
        if re.match(r"^\.LBB\d+_\d+:", ln) or re.match(r"^; %bb\.\d+:", ln):
            m = re.search(r"Depth=(\d+)", ln)
            depth = int(m.group(1)) if m else 0
        elif depth >= 2 and re.search(r"\bscratch_(load|store)", ln):
            in_loop_scratch += 1
    assert in_loop_scratch == 0, f"{in_loop_scratch} scratch accesses inside the step loop"
    assert re.search(r"Depth=2", text), "no nested loop found (the check would be vacuous)"
    assert re.search(r"v_mfma_f32_32x32x64_f8f6f4 v\[", text), "score MFMAs do not accumulate in VGPRs"
    assert len(re.findall(r"v_mfma_scale_f32_32x32x64_f8f6f4 a\[", text)) >= 16, "values MFMAs not in AGPRs"


def _kernel_loop_scratch(src, kernel_substr):
    """Scratch accesses inside loops (any depth) of one kernel of a source
    file, from the compiler's own loop annotations."""
    import re
    import shutil
    import tempfile

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = Path(d) / "k.s"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-I", str(CSRC), "-I", str(CSRC.parents[1] / "include"),
                        "-x", "hip", "--cuda-device-only", "-S", str(CSRC / src), "-o", str(out)],
                       check=True, capture_output=True)
        text = out.read_text()
    found, loops, in_loop_scratch, depth, inside = False, 0, 0, 0, False
    for ln in text.splitlines():
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            inside = kernel_substr in m.group(1)
            found |= inside
            depth = 0
            continue
        if not inside:
            continue
        if re.match(r"^\.LBB\d+_\d+:", ln) or re.match(r"^; %bb\.\d+:", ln):
            m = re.search(r"Depth=(\d+)", ln)
            depth = int(m.group(1)) if m else 0
            loops += depth > 0
        elif depth >= 1 and re.search(r"\bscratch_(load|store)", ln):
            in_loop_scratch += 1
    assert found, f"no kernel matching {kernel_substr} in {src}"
    assert loops > 0, "no loop found (the check would be vacuous)"
    return in_loop_scratch


@pytest.mark.parametrize("kernel", ["kv_expand_kernelILb0E", "kv_expand_kernelILb1E", "attn_expanded_kernel"])
def test_expanded_prefill_kernels_do_not_spill_in_loops(kernel):
    """The expanded-form prefill kernels keep their accumulators and staging
    in registers: no scratch traffic inside their stage / tile loops."""
    assert _kernel_loop_scratch("prefill_expanded.hip", kernel) == 0
