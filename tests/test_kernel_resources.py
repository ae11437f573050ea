"""Register and scratch use of every gfx950 kernel, from the compiler's resource report.

The attention kernels keep their accumulators, fragments and softmax state in
registers; an array indexed with a run-time value (or a spill) moves them to
per-lane scratch memory, which costs several times the pass's time without
changing its results, so no parity test notices.  Compiles the kernels for
gfx950 on the CPU (device code only) and requires, for every kernel, zero
bytes of scratch and no spilled VGPRs; SGPR spills, which go to VGPR lanes,
are allowed.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from cached_attention_amd import build

HIPCC = build.hipcc()


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_no_kernel_uses_scratch_or_spills_vgprs():
    src = os.path.join(build.CSRC, "fb_kernels.hip")
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [HIPCC, *build.HIPCC_FLAGS, f"-I{build.INCLUDE}", f"-I{build.CSRC}", "--cuda-device-only", "-c",
               "-o", os.path.join(tmp, "k.o"), src, "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = {}
    name = None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|VGPRs): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    attn = [k for k in kernels if "attn_bf16" in k]
    assert len(attn) >= 10, f"expected the bf16 attention configurations in the report, got {sorted(kernels)}"
    assert any("attn_f32m" in k for k in kernels) and any("combine_kernel" in k for k in kernels)
    bad = {k: v for k, v in kernels.items()
           if v.get("ScratchSize [bytes/lane]", 0) != 0 or v.get("VGPRs Spill", 0) != 0}
    assert not bad, f"kernels using scratch or spilling VGPRs: {bad}"
    # every kernel fits the 512-register file with at least one wave per SIMD
    assert all(v.get("VGPRs", 0) <= 512 for v in kernels.values())
