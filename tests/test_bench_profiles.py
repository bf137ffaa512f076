"""Host logic of the bench line: a committed counter summary is used only
while it was taken on the current kernel source and shared headers; any
change to either makes the figure unavailable (reported as null)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_summary_used_only_on_matching_source(tmp_path, monkeypatch):
    csrc = tmp_path / "block_scaled_fp4_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel v1\n")
    (csrc / "shared.h").write_text("header v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    h = bench.source_hash("k.hip")
    (prof / "k_traffic.txt").write_text(f"# summary\nkernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("k", "k.hip") == 1234.0
    # a changed kernel file or a changed header invalidates the summary
    (csrc / "k.hip").write_text("kernel v2\n")
    assert bench.read_traffic("k", "k.hip") is None
    (csrc / "k.hip").write_text("kernel v1\n")
    assert bench.read_traffic("k", "k.hip") == 1234.0
    (csrc / "shared.h").write_text("header v2\n")
    assert bench.read_traffic("k", "k.hip") is None
    # a missing summary or a missing figure is null too
    assert bench.read_profile("absent.txt", "k.hip", "x") is None
    assert bench.read_profile("k_traffic.txt", "k.hip", "no_such_key") is None
