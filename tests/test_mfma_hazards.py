"""The build-time MFMA read-distance check: pinned on hand-written disassembly, then run over
the built objects (CPU only: it reads the code objects, it runs nothing)."""
import glob
import os

import pytest

from mamba_ssd_prefill_amd import mfma_hazards as mh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kernel(body):
    return "<k>:\n" + "\n".join("\t" + l if not l.startswith("<") else l for l in body) + "\n"


def _check(body):
    return mh.check_text(_kernel(body))


def test_straight_line_with_full_nop_passes():
    assert _check(["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0", "s_nop 7",
                   "v_accvgpr_read_b32 v8, a3", "s_endpgm"]) == []


def test_straight_line_one_short_fails():
    bad = _check(["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0", "s_nop 6",
                  "v_accvgpr_read_b32 v8, a3", "s_endpgm"])
    assert len(bad) == 1 and "7 wait states (needs 8)" in bad[0]


def test_fp32_mfma_needs_ten():
    body = ["v_mfma_f32_16x16x4_f32 v[0:3], v8, v9, 0", "s_nop 8", "v_add_f32_e32 v10, v3, v3", "s_endpgm"]
    assert len(_check(body)) == 1
    body[1] = "s_nop 9"
    assert _check(body) == []


def test_short_side_of_a_branch_is_found():
    # the long side has 8 instructions before the join, the short side 2: only the latter is short
    body = ["v_mfma_f32_16x16x32_bf16 a[16:19], v[0:3], v[4:7], a[16:19]",
            "s_cbranch_vccnz L1"] + ["v_mov_b32_e32 v%d, 0" % (20 + i) for i in range(8)] + [
            "<L1>:", "s_mov_b64 s[6:7], -1", "v_accvgpr_read_b32 v9, a19", "s_endpgm"]
    bad = _check(body)
    assert len(bad) == 1 and "after 2 wait states" in bad[0]


def test_accumulation_chain_is_not_a_read_but_an_early_overwrite_is():
    assert _check(["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0",
                   "v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[4:7], a[0:3]", "s_nop 7",
                   "v_accvgpr_read_b32 v12, a0", "s_endpgm"]) == []
    assert _check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
                   "v_mfma_f32_16x16x32_bf16 v[12:15], v[16:19], v[8:11], v[0:3]", "s_nop 7",
                   "v_add_f32_e32 v30, v12, v13", "s_endpgm"]) == []
    assert len(_check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                       "v_mfma_f32_16x16x32_bf16 v[12:15], v[16:19], v[8:11], v[2:5]", "s_endpgm"])) == 1
    assert len(_check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                       "v_mov_b64_e32 v[0:1], v[20:21]", "s_endpgm"])) == 1
    # past the distance, nothing is tracked any more
    assert _check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0", "s_nop 7",
                   "v_mov_b64_e32 v[0:1], v[20:21]", "v_add_f32_e32 v30, v0, v1", "s_endpgm"]) == []


def test_load_into_result_registers_is_not_a_read():
    assert _check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                   "ds_read_b128 v[0:3], v20 offset:16", "s_endpgm"]) == []
    assert len(_check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                       "ds_read_b128 v[12:15], v2 offset:16", "s_endpgm"])) == 1


def test_operand_and_store_reads_are_found():
    assert len(_check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                       "v_mfma_f32_16x16x32_bf16 v[12:15], v[0:3], v[8:11], 0", "s_endpgm"])) == 1
    assert len(_check(["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                       "buffer_store_dwordx4 v[0:3], v20, s[4:7], 0 offen", "s_endpgm"])) == 1


def test_unknown_mfma_is_refused():
    with pytest.raises(ValueError):
        _check(["v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], 0", "s_endpgm"])


def test_built_objects_are_clean():
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    if not objs:
        pytest.skip("library not built")
    assert mh.check_objects(objs) == []


def test_registers_an_accumulation_chain_overwrote_are_not_tracked():
    # the second MFMA accumulates onto the first's result and writes part of it anew; the third
    # reads that part as its C: a read of the second's result, chained, not of the first's
    assert _check(["v_mfma_f32_16x16x32_f16 v[56:59], v[110:113], v[74:77], v[62:65]",
                   "v_mfma_f32_16x16x32_f16 v[54:57], v[106:109], v[86:89], v[56:59]",
                   "v_mfma_f32_16x16x32_f16 v[30:33], v[114:117], v[94:97], v[54:57]", "s_endpgm"]) == []
