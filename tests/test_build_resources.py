"""Compiler resource report of every kernel in the library (CPU only: hipcc cross-compiles
for gfx950).

A kernel that takes its argument block by value copies it to per-lane scratch memory as
soon as a device function that receives the block by reference is not inlined; the
launch then reserves scratch for every lane and slows down by microseconds. No kernel
of the library may use scratch (spills included)."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_no_kernel_uses_scratch(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from certified_sparse_attention_amd import _build
    cmd = [hipcc] + [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")] + [
        "-c", "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
        "-I", os.path.join(ROOT, "include"), "-o", str(tmp_path / "dev.o"),
        os.path.join(ROOT, "certified_sparse_attention_amd", "csrc", "api.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    report = {}
    name = None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            report[name] = int(m.group(1))
    kernels = {k: v for k, v in report.items() if "kernel" in k}
    assert len(kernels) >= 8, report
    assert all(v == 0 for v in kernels.values()), {k: v for k, v in kernels.items() if v}
