"""Host logic of bench.py (CPU only): the multi-GPU refusal and the digest gate
on the measured traffic taken from a committed profile summary."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _profile(tmp_path, monkeypatch, sources, prefix, traffic="123456"):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    (prof / "p.md").write_text(
        f"# summary\n\ntraffic_bytes_per_launch: {traffic}\nkernel_sources: {' '.join(sources)}\n"
        f"kernel_sources_sha256_prefix: {prefix}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return "p.md"


def test_traffic_reported_while_sources_match(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_text("kernel a\n")
    (tmp_path / "b.h").write_text("header b\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.sources_digest(["a.hip", "b.h"])
    name = _profile(tmp_path, monkeypatch, ["a.hip", "b.h"], digest[:16])
    assert bench.measured_traffic(name) == 123456


@pytest.mark.parametrize("change", ["a.hip", "b.h"])
def test_traffic_dropped_when_a_source_changes(tmp_path, monkeypatch, change):
    (tmp_path / "a.hip").write_text("kernel a\n")
    (tmp_path / "b.h").write_text("header b\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.sources_digest(["a.hip", "b.h"])
    name = _profile(tmp_path, monkeypatch, ["a.hip", "b.h"], digest[:16])
    (tmp_path / change).write_text("edited\n")
    assert bench.measured_traffic(name) is None


def test_traffic_kept_across_comment_edits_only(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_text("int f(int x) { return x + 1; }  // add one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.sources_digest(["a.hip"])
    name = _profile(tmp_path, monkeypatch, ["a.hip"], digest[:16])
    (tmp_path / "a.hip").write_text("/* increment */\nint f(int x) {\n  return x + 1;   // one more\n}\n")
    assert bench.measured_traffic(name) == 123456
    (tmp_path / "a.hip").write_text("int f(int x) { return x + 2; }  // add one\n")
    assert bench.measured_traffic(name) is None


def test_traffic_missing_profile_is_none(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("absent.md") is None


def test_committed_profiles_name_existing_sources():
    # every committed W1 summary names its kernel sources, and they exist
    for name in bench.PROFILES.values():
        path = os.path.join(ROOT, "profiles", name)
        fields = {}
        for line in open(path):
            key, sep, val = line.partition(":")
            if sep:
                fields[key] = val.strip()
        if "kernel_sources" not in fields:
            continue   # a summary from before the digest covered every source
        for src in fields["kernel_sources"].split():
            assert os.path.exists(os.path.join(ROOT, src)), src
