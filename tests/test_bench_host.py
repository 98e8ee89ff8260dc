"""Host-side checks of bench.py (no GPU): the one-GPU contract and the rule that a committed traffic figure is
used only while the kernel sources still hash to the value recorded with the counters."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_summary(tmp_path, kind, config, T, sha, traffic):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    (prof / f"hbm_traffic_{kind}_{config}_T{T}.md").write_text(
        f"# summary\n\n    source_sha256: {sha}\n    traffic_bytes_per_launch: {traffic}\n")


def _sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "routed_expert_ffn_sigmoid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


@pytest.mark.parametrize("gemm,files", [(False, ("ffn_decode.hip", "common.h", "kernels.h")),
                                        (True, ("ffn_gemm.hip", "common.h", "kernels.h"))])
def test_traffic_follows_the_source_hash(tmp_path, monkeypatch, gemm, files):
    kind = "gemm" if gemm else "decode"
    # a copy of the sources next to a summary, so the check runs on files this test controls
    csrc = tmp_path / "routed_expert_ffn_sigmoid_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in files:
        with open(os.path.join(ROOT, "routed_expert_ffn_sigmoid_amd", "csrc", f), "rb") as fh:
            (csrc / f).write_bytes(fh.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", 7, gemm) is None  # no summary
    _write_summary(tmp_path, kind, "wl", 7, _sources_sha(files), 123456)
    assert bench.measured_traffic("wl", 7, gemm) == 123456.0
    (csrc / files[0]).write_bytes((csrc / files[0]).read_bytes() + b"\n// edited\n")
    assert bench.measured_traffic("wl", 7, gemm) is None  # sources changed since the counters
