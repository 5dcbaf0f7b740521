"""Resource use of the gfx950 decode kernels, read from the compiler's own
metadata (hipcc -S of the kernel source, device only): no register spills
to scratch memory, no private segment, and at most 64 VGPRs, so that two
1024-lane workgroups (8 waves per SIMD) stay resident per CU.  CPU only."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "lossless_entropy_coded_huffman_amd", "csrc", "dfh_decode.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "decode.s")
    subprocess.check_call([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
                           "--cuda-device-only", "-S", SRC, "-o", out], stderr=subprocess.DEVNULL)
    text = open(out).read()
    meta = {}
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        if "decode_kernel" not in name:
            continue
        meta[name] = {k: int(re.search(r"\.%s:\s+(\d+)" % k, block).group(1))
                      for k in ("private_segment_fixed_size", "vgpr_count", "vgpr_spill_count")}
    return meta


def test_twelve_decode_kernels(kernels):
    # three kinds, checked and unchecked, at raised and base wave priority
    assert len(kernels) == 12


def test_no_scratch_and_64_vgprs(kernels):
    for name, m in kernels.items():
        assert m["private_segment_fixed_size"] == 0, (name, m)
        assert m["vgpr_spill_count"] == 0, (name, m)
        assert m["vgpr_count"] <= 64, (name, m)
