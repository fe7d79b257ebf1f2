"""Register budget of the streaming kernels, checked at build time without a
GPU: hipcc's kernel resource-usage remarks for gfx950 must show no register
spills in any forward or fused-backward instantiation.  A spill inside the
row loop costs more than anything else in these kernels (it turned a 32 us
forward into a 52 us one)."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "adaln_fwd_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    """Spilled VGPRs per kernel of fwd.hip, fwd_wide.hip, bwd_fused.hip and
    bwd_wide.hip (compiled in parallel)."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("res")
    procs = {}
    for src in ("fwd.hip", "fwd_wide.hip", "bwd_fused.hip", "bwd_wide.hip"):
        procs[src] = subprocess.Popen(
            [HIPCC, "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"),
             "-Rpass-analysis=kernel-resource-usage", "-c",
             os.path.join(CSRC, src), "-o", str(tmp / (src + ".o"))],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    out = {}
    for src, p in procs.items():
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-2000:]
        spills = {}
        for block in err.split("remark: Function Name: ")[1:]:
            name = block.split("\n", 1)[0].strip()
            m = re.search(r"VGPRs Spill: (\d+)", block)
            spills[name] = int(m.group(1)) if m else 0
        out[src] = spills
    return out


def test_forward_row_kernels_do_not_spill(usage):
    stream = {k: v for k, v in usage["fwd.hip"].items()
              if "fwd_rows_kernel" in k}
    assert len(stream) >= 80
    spills = {k: v for k, v in stream.items() if v}
    assert not spills, spills


def test_backward_stream_kernels_do_not_spill(usage):
    stream = {k: v for k, v in usage["bwd_fused.hip"].items()
              if "bwd_stream_kernel" in k}
    assert len(stream) >= 32
    spills = {k: v for k, v in stream.items() if v}
    assert not spills, spills


def test_wide_backward_kernels_do_not_spill(usage):
    wide = {k: v for k, v in usage["bwd_wide.hip"].items()
            if "bwd_wide_kernel" in k}
    assert len(wide) >= 24
    spills = {k: v for k, v in wide.items() if v}
    assert not spills, spills


def test_forward_wide_kernels_do_not_spill(usage):
    """The forward of rows past 1024 vectors (pairs and quads of
    wavefronts), the 16-vector rows included."""
    wide = {k: v for k, v in usage["fwd_wide.hip"].items()
            if "fwd_wide_kernel" in k}
    assert len(wide) >= 24
    spills = {k: v for k, v in wide.items() if v}
    assert not spills, spills