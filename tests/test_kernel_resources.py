"""Register and LDS budgets of the device kernels (CPU: hipcc cross-compiles for gfx950).

The matrix-core kernels hold their accumulators in registers and run one work-group of
512 threads per CU: a kernel that spills to scratch memory still computes the right
values, so no parity test notices, but it runs several times slower.  This test
compiles every HIP source for the device alone with the compiler's resource report and
checks that no kernel uses scratch memory, that none needs more than the 160 KiB of LDS
of a CU, and that no kernel exceeds the 512 registers (vector plus accumulation) that
one wave can hold.  The generic kernels (any head dim, one thread per query or key row,
names ending in _simple_kernel) keep a row's accumulators in a private array by design
and are exempt from the scratch check.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dag_packed_attention_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = ("kernels.hip", "gdn.hip", "logprob.hip", "conv.hip")


def _resources(src):
    """{kernel name: {field: value}} from hipcc's kernel-resource-usage remarks."""
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(CSRC, src),
               "-o", os.path.join(tmp, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES)
def test_no_kernel_spills_or_exceeds_the_cu(src):
    res = _resources(src)
    kernels = {k: v for k, v in res.items() if "ScratchSize" in v}
    assert kernels, f"no kernel-resource remarks parsed for {src}"
    for name, v in kernels.items():
        if "_simple_kernel" not in name:
            assert v["ScratchSize"] == 0, f"{name} spills {v['ScratchSize']} bytes per lane to scratch"
        assert v.get("LDS Size", 0) <= 160 * 1024, f"{name} needs {v['LDS Size']} bytes of LDS"
        assert v.get("VGPRs", 0) + v.get("AGPRs", 0) <= 512, f"{name} uses {v} registers"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_the_attention_kernels_are_reported():
    names = " ".join(_resources("kernels.hip"))
    for k in ("fwd_mfma_kernel", "dq_mfma_kernel", "dkdv_mfma_kernel", "dkdv_group_kernel"):
        assert k in names, k
