"""Static checks of the head-size-128 prefill kernel's gfx950 assembly (no GPU needed).

Its MFMAs are inline asm with hand-placed registers, so the compiler guards none of their
hazards and the fixed accumulator registers a0..a127 must never be touched by compiler code.
The kernel source is compiled to assembly here and scanned with tests/mfma_asm_check.py; a
hazard planted in a copy of that assembly shows that the scan finds it.
"""
import os
import re
import shutil
import subprocess

import pytest

from tests import mfma_asm_check as chk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_attention_08_amd", "csrc", "attn_fwd_d128.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNELS = [f"_ZN4attn12_GLOBAL__N_119prefill_d128_kernelILb{b}ELb{c}E"
           for b in (1, 0) for c in (1, 0)]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("d128") / "d128.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return out.read_text()


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_unguarded_mfma_hazards(asm, kernel):
    findings = chk.check(chk.kernel_body(asm, kernel))
    assert not findings, findings[:10]


@pytest.mark.parametrize("kernel", KERNELS)
def test_registers_fit_one_wave_per_simd_without_scratch(asm, kernel):
    end = asm.find(".Lfunc_end", asm.find(kernel + "EE"))
    tail = asm[end:end + 4000]
    num = lambda key: int(re.search(key + r":\s*(\d+)", tail).group(1))
    assert num("; ScratchSize") == 0
    assert num("; NumAgprs") >= chk.N_FIXED          # the fixed accumulators are counted
    assert num("; NumVgprs") <= 256 and num("; TotalNumVgprs") <= 512


def test_planted_hazards_are_found(asm):
    lines = chk.kernel_body(asm, KERNELS[0])
    assert not chk.check(lines)
    # drop the wait states that end every 32-key block: the next block's statistics then
    # read scores and accumulators too early
    cut = [l for l in lines if l.strip() not in ("s_nop 7", "s_nop 4")]
    assert any("after" in msg for _, msg in chk.check(cut))
    # a compiler instruction writing a fixed accumulator outside inline asm
    k = next(i for i, l in enumerate(lines) if l.strip().startswith("v_exp_f32"))
    planted = lines[:k] + ["\tv_accvgpr_write_b32 a5, v0"] + lines[k:]
    assert any("fixed accumulator" in msg for _, msg in chk.check(planted))
    # a vector result fed to an O^T MFMA (P, its B operand) without the two wait states
    m = next(i for i, l in enumerate(lines)
             if l.strip().startswith("v_mfma") and l.split()[1].startswith("a["))
    src_b = chk.split_ops(lines[m].split(None, 1)[1])[2]
    first = re.match(r"v\[(\d+):", src_b).group(1)
    planted = lines[:m] + [f"\tv_mov_b32 v{first}, 0"] + lines[m:]
    assert any("vector result" in msg for _, msg in chk.check(planted))
