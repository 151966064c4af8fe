"""MFMA data-hazard check of the attention kernels' gfx950 assembly, and pins of
the checker itself on hand-written cases (host only: hipcc cross-compiles)."""

import os
import shutil
import subprocess

import pytest

import mfma_hazards as mh

from streaming_causal_video_amd import build as B

KERNELS = ["attn_bf16.hip", "attn_fp8.hip"]


def _asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [B.hipcc(), *B.CFLAGS, *B.EXTRA.get(src, []), "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_kernel_assembly_has_no_mfma_hazards(src, tmp_path):
    text = _asm(src, tmp_path)
    assert "v_mfma" in text
    found = mh.check(text)
    assert not found, "\n".join(found[:10])


def _fn(body):
    return "\t.type\tk,@function\nk:\n" + body + "\ts_endpgm\n.Lfunc_end0:\n"


MFMA = "\tv_mfma_f32_32x32x16_bf16 {d}, v[0:3], v[4:7], {c}\n"


def test_checker_flags_early_read_of_result():
    text = _fn(MFMA.format(d="a[0:15]", c="a[0:15]") + "\tv_accvgpr_read_b32 v10, a3\n")
    assert len(mh.check(text)) == 1


def test_checker_accepts_read_after_enough_wait_states():
    text = _fn(MFMA.format(d="v[16:31]", c="0") + "\ts_nop 7\n\ts_nop 3\n"
               + "\tv_add_f32_e32 v40, v16, v17\n")
    assert mh.check(text) == []
    text = _fn(MFMA.format(d="v[16:31]", c="0") + "\ts_nop 7\n\ts_nop 2\n"
               + "\tv_add_f32_e32 v40, v16, v17\n")
    assert len(mh.check(text)) == 1


def test_checker_allows_back_to_back_accumulation_only_on_the_same_registers():
    same = MFMA.format(d="v[16:31]", c="0") + MFMA.format(d="v[16:31]", c="v[16:31]")
    assert mh.check(_fn(same)) == []
    part = MFMA.format(d="v[16:31]", c="0") + MFMA.format(d="v[32:47]", c="v[20:35]")
    assert len(mh.check(_fn(part))) == 1


def test_checker_flags_overwrite_of_accumulator_input():
    # the MFMA reads srcC v[16:31] (written long before); a VALU write to it right after
    body = "\tv_mov_b32_e32 v16, 0\n\ts_nop 7\n\ts_nop 7\n" + MFMA.format(d="v[48:63]", c="v[16:31]")
    assert mh.check(_fn(body + "\ts_nop 7\n\tv_mov_b32_e32 v17, 1\n")) == []
    assert len(mh.check(_fn(body + "\tv_mov_b32_e32 v17, 1\n"))) == 1


def test_checker_flags_valu_write_feeding_mfma():
    body = "\tv_mov_b32_e32 v5, 0\n" + MFMA.format(d="v[16:31]", c="0")
    assert len(mh.check(_fn(body))) == 1
    body = "\tv_mov_b32_e32 v5, 0\n\ts_nop 1\n" + MFMA.format(d="v[16:31]", c="0")
    assert mh.check(_fn(body)) == []


def test_checker_follows_loop_back_edges():
    # the read at the loop head is far from the MFMA in text order but one
    # instruction after it along the back edge
    body = (".LBB0_1:\n\tv_add_f32_e32 v40, v16, v17\n" + "\ts_nop 7\n" * 3
            + MFMA.format(d="v[16:31]", c="0") + "\ts_cbranch_scc1 .LBB0_1\n")
    assert len(mh.check(_fn(body))) == 1


def test_checker_windows_follow_the_pass_count():
    assert mh.mfma_passes("v_mfma_f32_16x16x32_bf16") == 4
    assert mh.mfma_passes("v_mfma_f32_32x32x16_bf16") == 8
    assert mh.mfma_passes("v_mfma_scale_f32_32x32x64_f8f6f4") == 16
    assert mh.mfma_passes("v_mfma_f32_32x32x64_f8f6f4") == 16
    short = "\tv_mfma_f32_16x16x32_bf16 v[16:19], v[0:3], v[4:7], 0\n"
    # a 4-pass result may be read 8 wait states after issue, not 7
    assert mh.check(_fn(short + "\ts_nop 7\n\tv_add_f32_e32 v40, v16, v17\n")) == []
    assert len(mh.check(_fn(short + "\ts_nop 6\n\tv_add_f32_e32 v40, v16, v17\n"))) == 1
    # the same spacing is too short for an 8-pass result
    assert len(mh.check(_fn(MFMA.format(d="v[16:31]", c="0")
                            + "\ts_nop 7\n\tv_add_f32_e32 v40, v16, v17\n"))) == 1


def test_checker_16_pass_result_window_is_19():
    long = "\tv_mfma_f32_32x32x64_f8f6f4 v[16:31], v[0:7], v[8:15], 0\n"
    assert mh.check(_fn(long + "\ts_nop 15\n\ts_nop 2\n\tv_add_f32_e32 v40, v16, v17\n")) == []
    assert len(mh.check(_fn(long + "\ts_nop 15\n\ts_nop 1\n\tv_add_f32_e32 v40, v16, v17\n"))) == 1
