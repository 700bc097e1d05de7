"""bench.py's host logic on the CPU: the one-GPU contract, the committed
counter summary it reads, and the source hash that ties the two together."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_forward_source_hash_covers_the_forward_sources(tmp_path, monkeypatch):
    h = bench.forward_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    # a copy of the sources hashes the same; one changed byte changes it
    for rel in bench.FWD_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.forward_source_hash() == h
    last = tmp_path / bench.FWD_SOURCES[-1]
    last.write_bytes(last.read_bytes() + b"\n")
    assert bench.forward_source_hash() != h


def _summary(root, sha, traffic):
    path = os.path.join(root, bench.PMC_SUMMARY)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write("counter summary\n\n")
        if sha is not None:
            fh.write(f"source_sha256: {sha}\n")
        if traffic is not None:
            fh.write(f"traffic_bytes_per_launch: {traffic}\n")


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    for rel in bench.FWD_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return str(tmp_path)


def test_traffic_is_read_for_the_current_sources_only(fake_root):
    sha = bench.forward_source_hash()
    _summary(fake_root, sha, "8.911e+09")
    assert bench.measured_traffic("720p") == pytest.approx(8.911e9)
    # taken on other code, for another workload, or incomplete: no figure
    assert bench.measured_traffic("1080p") is None
    _summary(fake_root, "0" * 16, "8.911e+09")
    assert bench.measured_traffic("720p") is None
    _summary(fake_root, sha, None)
    assert bench.measured_traffic("720p") is None
    _summary(fake_root, None, "8.911e+09")
    assert bench.measured_traffic("720p") is None
    os.remove(os.path.join(fake_root, bench.PMC_SUMMARY))
    assert bench.measured_traffic("720p") is None


def test_committed_summary_is_well_formed():
    text = open(os.path.join(ROOT, bench.PMC_SUMMARY)).read()
    assert "source_sha256:" in text and "traffic_bytes_per_launch:" in text
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
