"""Host logic of bench.py that needs no GPU: the digest that ties the committed
HBM-traffic counters to the FFN kernel code they were taken with."""
import json
import os
import shutil

import bench


def _copy_sources(tmp_path):
    for f in bench.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, f), dst)


def _digest_at(monkeypatch, root):
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench.kernel_source_digest()


def test_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    base = _digest_at(monkeypatch, tmp_path)
    f = tmp_path / bench.KERNEL_SOURCES[0]
    text = f.read_text()
    f.write_text("// a new line comment\n/* and a\n   block comment */\n" + text.replace("\n", "\n\n", 3) + "\n   \n")
    assert _digest_at(monkeypatch, tmp_path) == base


def test_digest_changes_with_the_code(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    base = _digest_at(monkeypatch, tmp_path)
    f = tmp_path / bench.KERNEL_SOURCES[1]
    f.write_text(f.read_text() + "\nstatic const int unused_constant = 1;\n")
    assert _digest_at(monkeypatch, tmp_path) != base


def test_traffic_is_reported_only_for_the_code_it_was_taken_with(tmp_path, monkeypatch):
    traffic = {"kernel_source_sha256": bench.kernel_source_digest(), "fetch_factor": 2.0, "write_factor": 1.0,
               "kernels": {"decode/ffn_up": {"fetch_kib": 100.0, "write_kib": 10.0}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(traffic))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("decode", "ffn_up") == int((100.0 * 2.0 + 10.0 * 1.0) * 1024)
    assert bench.measured_traffic("decode", "ffn_down") is None
    traffic["kernel_source_sha256"] = "0" * 64
    path.write_text(json.dumps(traffic))
    assert bench.measured_traffic("decode", "ffn_up") is None
