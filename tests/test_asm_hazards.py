"""The hand-placed wait states around the kernels' inline-asm matrix products,
checked on the gfx950 assembly the build keeps (CPU only), and the checker
itself on planted hazards."""

import glob
import os

import pytest

import asm_lint

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_kv_cache_paged_amd")
ASM_DIR = os.path.join(PKG, "_asm")
HIP_SOURCES = sorted(os.path.basename(p) for p in glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _fresh():
    if not all(os.path.exists(os.path.join(ASM_DIR, s + ".s")) for s in HIP_SOURCES):
        return False
    newest_src = max(os.path.getmtime(p) for p in glob.glob(os.path.join(PKG, "csrc", "*")))
    return min(os.path.getmtime(os.path.join(ASM_DIR, s + ".s")) for s in HIP_SOURCES) >= newest_src


@pytest.fixture(scope="module")
def asm_files():
    if not _fresh():
        from fp8_kv_cache_paged_amd import _build
        _build.build()
    return {s: open(os.path.join(ASM_DIR, s + ".s")).read() for s in HIP_SOURCES}


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_library_assembly_keeps_the_wait_states(asm_files, src):
    nfunc, violations = asm_lint.check_text(asm_files[src])
    assert not violations, "\n".join(violations[:20])


def test_every_decode_kernel_is_checked(asm_files):
    names = [n for text in asm_files.values() for n in asm_lint.parse_functions(text)]
    for kernel in ("mla_decode_ws_kernel", "mla_decode_kernel", "mla_decode_rows_kernel", "mla_combine_kernel",
                   "kv_encode_kernel"):
        assert any(kernel in n for n in names), kernel
    assert len(names) >= 100


def test_every_matrix_product_form_is_known(asm_files):
    for src, text in asm_files.items():
        for name, items in asm_lint.parse_functions(text).items():
            for kind, x in items:
                if kind == "insn" and x.op.startswith("v_mfma"):
                    assert x.op in asm_lint.MFMA_PASSES, f"{src}: {name}: {x.op}"


def _fn(body):
    return "\t.text\nk:\n" + "".join(f"\t{line}\n" for line in body) + ".Lfunc_end0:\n"


MF8 = "v_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15]"
BF16 = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"


@pytest.mark.parametrize("body,bad", [
    ([MF8, "v_mov_b32_e32 v40, v3", "s_endpgm"], True),                                  # read at once
    ([MF8, "s_nop 7", "s_nop 7", "s_nop 2", "v_mov_b32_e32 v40, v3", "s_endpgm"], True),   # 19 < 20
    ([MF8, "s_nop 7", "s_nop 7", "s_nop 3", "v_mov_b32_e32 v40, v3", "s_endpgm"], False),  # 20
    ([MF8, "v_mov_b32_e32 v40, v41", "s_endpgm"], False),                                # other registers
    ([MF8, "ds_write_b128 v50, v[4:7]", "s_endpgm"], True),                              # stored too early
    ([MF8, "ds_read_b128 v[8:11], v50", "s_endpgm"], True),                              # overwritten
    ([MF8, MF8, "s_endpgm"], False),                                                     # accumulator forwarded
    ([MF8, "v_mfma_f32_32x32x64_f8f6f4 v[32:47], v[0:7], v[24:31], v[32:47]", "s_endpgm"], True),  # as A
    (["v_mov_b32_e32 v17, 0", MF8, "s_endpgm"], True),                                   # VALU -> A
    (["v_mov_b32_e32 v17, 0", "s_nop 1", MF8, "s_endpgm"], False),
    (["v_mul_f32_e32 v3, v3, v9", "s_nop 0", BF16, "s_endpgm"], True),                  # VALU -> C, 1 slot
    ([BF16, "s_nop 7", "s_nop 3", "v_mov_b32_e32 v40, v3", "s_endpgm"], False),         # 12 for 8 passes
    ([BF16, "s_nop 7", "s_nop 2", "v_mov_b32_e32 v40, v3", "s_endpgm"], True),
])
def test_checker_on_planted_hazards(body, bad):
    n, v = asm_lint.check_text(_fn(body))
    assert n == 1
    assert bool(v) == bad, v


def test_checker_follows_branches_and_loops():
    # the product at the loop's end reaches the read at its head through the back edge
    loop = _fn(["s_mov_b32 s0, 4", ".LBB0_1:", "v_add_f32_e32 v40, v3, v3", MF8, "s_sub_u32 s0, s0, 1",
                "s_cbranch_scc1 .LBB0_1", "s_endpgm"])
    loop = loop.replace("\t.LBB0_1:\n", ".LBB0_1:\n")
    n, v = asm_lint.check_text(loop)
    assert v and "v3" in v[0]
    # one path with the wait, one without: the join keeps the worst
    join = _fn([MF8, "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7", "s_nop 7", ".LBB0_2:",
                "v_mov_b32_e32 v40, v3", "s_endpgm"]).replace("\t.LBB0_2:\n", ".LBB0_2:\n")
    assert asm_lint.check_text(join)[1]


def test_checker_rejects_forbidden_classes():
    packed = "v_pk_" + "add_f32 v[0:1], v[2:3], v[4:5]"
    assert asm_lint.check_text(_fn([packed, "s_endpgm"]))[1]
    scal = "s_" + "st" + "ore_dword s0, s[2:3], 0x0"
    assert asm_lint.check_text(_fn([scal, "s_endpgm"]))[1]
