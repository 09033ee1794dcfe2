"""Host-side logic of bench.py (no GPU): the keys that tie the committed
rocprofv3 traffic figures to the kernel sources, and the one-GPU guard."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _tree(tmp_path):
    """A copy of the kernel sources and the public header under tmp_path."""
    for sub in (os.path.join("combine_experts_amd", "csrc"), "include"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub)
    return tmp_path


def test_source_digest_covers_included_headers_not_comments(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    base = {f: bench.source_digest(f) for f in ("gemm_tiled.hip", "ffn.hip")}
    assert base == {f: bench.source_digest(f) for f in base}  # deterministic
    csrc = root / "combine_experts_amd" / "csrc"
    # comments, blank lines and indentation do not change a key
    with open(csrc / "ffn_body.h", "a") as fh:
        fh.write("\n// a comment\n/* another\n   comment */\n\n   \n")
    with open(csrc / "gemm_tiled.hip", "a") as fh:
        fh.write("\n\n  // a comment\n")
    assert {f: bench.source_digest(f) for f in base} == base
    # code in a header only ffn.hip includes (through ffn_body.h) changes its key alone
    with open(csrc / "ffn_body.h", "a") as fh:
        fh.write("\nstatic const int edited_marker = 1;\n")
    assert bench.source_digest("ffn.hip") != base["ffn.hip"]
    assert bench.source_digest("gemm_tiled.hip") == base["gemm_tiled.hip"]
    # the public header, included by both through moe_kernels.h / moe_device.h
    with open(root / "include" / "moe.h", "a") as fh:
        fh.write("\ntypedef int edited_marker_t;\n")
    assert bench.source_digest("gemm_tiled.hip") != base["gemm_tiled.hip"]
    # a source neither includes changes neither key
    before = bench.source_digest("gemm_tiled.hip")
    with open(csrc / "combine.hip", "a") as fh:
        fh.write("\nstatic const int edited_marker = 2;\n")
    assert bench.source_digest("gemm_tiled.hip") == before


def test_committed_traffic_matches_the_current_sources():
    """The headline gate/up launch (and its down pass) have HBM traffic
    figures taken on the sources as they are; a kernel or header change
    without new counters shows up here as a missing figure."""
    for key in ("gate_up deepseek-v3-moe-prefill-zipf T=4096", "down deepseek-v3-moe-prefill-zipf T=4096"):
        t = bench.kernel_traffic(key, "gemm_tiled.hip")
        assert t is not None and t > 1e9, key
    assert bench.kernel_traffic("gate_up deepseek-v3-moe-decode-fp8 T=512", "ffn.hip") is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
