"""The gfx950 kernels keep every per-lane array in registers: no scratch
memory and no VGPR spills (either would put global-memory traffic on the hot
loop).  Compiles the kernel source with hipcc's resource-usage remarks; CPU only."""
import re
import shutil
import subprocess

import pytest

from exact_attention_forward_02_amd import build


def _remarks(source):
    cmd = [build.hipcc(), *[f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")],
           *build.source_flags(source), "-c", source, "-o", "/dev/null",
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True)
    return out.stderr


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not build.hipcc().startswith("/"),
                    reason="hipcc not available")
def test_no_scratch_and_no_vgpr_spills():
    text = _remarks(build.SOURCES[0])
    kernels = re.findall(r"Function Name: (\S+)", text)
    # 3 head-dim pairs x causal or not x (bf16, bf16 debug, fp16, bf16 packed varlen),
    # plus the chained-sweep forms of the non-causal bf16, debug and fp16 kernels at
    # equal head dims (64, 64) and (128, 128)
    assert len(kernels) == 24 + 2 * 3, f"expected 30 kernel instantiations, found {len(kernels)}"
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", text)]
    occupancy = [int(x) for x in re.findall(r"Occupancy \[waves/SIMD\]: (\d+)", text)]
    assert len(scratch) == len(kernels) and all(s == 0 for s in scratch), scratch
    assert all(s == 0 for s in spills), spills
    # one 8-wave workgroup per CU needs two waves per SIMD
    assert all(o >= 2 for o in occupancy), occupancy


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not build.hipcc().startswith("/"),
                    reason="hipcc not available")
def test_merge_kernel_resources():
    text = _remarks(build.SOURCES[1])
    kernels = re.findall(r"Function Name: (\S+)", text)
    assert len(kernels) == 2, kernels
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    assert scratch == [0, 0], scratch


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not build.hipcc().startswith("/"),
                    reason="hipcc not available")
def test_decode_kernel_resources():
    text = _remarks(build.SOURCES[3])
    kernels = re.findall(r"Function Name: (\S+)", text)
    assert len(kernels) == 6, kernels  # (64,64), (128,128), (192,128) x causal or not
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", text)]
    assert scratch == [0] * 6 and spills == [0] * 6, (scratch, spills)


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not build.hipcc().startswith("/"),
                    reason="hipcc not available")
def test_backward_kernel_resources():
    text = _remarks(build.SOURCES[2])
    kernels = re.findall(r"Function Name: (\S+)", text)
    # per element type (bf16, fp16): D for d_v = 64, 128; dK/dV and dQ for (64,64) and
    # (128,128), causal or not; (192,128) with dK/dV as two passes (dV, then dK)
    assert len(kernels) == 2 * (2 + 2 * 2 + 2 * 2 + 2 * 3), kernels
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", text)]
    assert scratch == [0] * len(kernels) and spills == [0] * len(kernels), (scratch, spills)
