"""The compiler's own resource report for the bf16 GEMM kernels (host-only: a device-only
compile for gfx950 with -Rpass-analysis=kernel-resource-usage, no GPU).  The logits, recompute,
kept-logits and dH GEMMs hold 256 fp32 accumulators per lane next to their operand registers at
one wave per SIMD; a spill there puts scratch traffic into the epilogue or the main loop, so
every one of their variants must compile without spills or scratch."""
import os
import re
import subprocess

import pytest

from rl_fine_tuning_amd import build as B

# gemm16_kernel<KIND, ...>: 0 logits + LSE, 1 recompute (probabilities), 2 dH on row-major W,
# 3 dH on the fragment-major W^T, 4 logits keeping the chunk's logits, 5 dW
SPILL_FREE_KINDS = {0, 1, 2, 3, 4}


def _report():
    cmd = [B.hipcc(), *[f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "--offload-device-only", "-c",
           "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC,
           os.path.join(B.CSRC, "grpo_kernels.hip"), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = {}
    for block in re.split(r"remark: Function Name: ", res.stderr)[1:]:
        name = block.split()[0]
        fields = dict(re.findall(r"remark:\s+(\w[\w /\[\]]*?): (\w+) \[-Rpass", block))
        kernels[name] = fields
    return kernels


def _have_hipcc():
    try:
        B.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not installed")
def test_gemm_kernels_do_not_spill():
    kernels = _report()
    gemm = {n: f for n, f in kernels.items() if "gemm16_kernel" in n}
    assert gemm, "no bf16 GEMM kernel in the resource report"
    checked = 0
    for name, f in gemm.items():
        kind = int(re.search(r"gemm16_kernelILi(\d+)E", name).group(1))
        if kind not in SPILL_FREE_KINDS:
            continue
        checked += 1
        assert int(f.get("VGPRs Spill", -1)) == 0, (name, f)
        assert int(f.get("SGPRs Spill", -1)) == 0, (name, f)
        assert int(f.get("ScratchSize [bytes/lane]", -1)) == 0, (name, f)
        assert int(f.get("Occupancy [waves/SIMD]", 1)) >= 1, (name, f)
    assert checked >= 15, checked
