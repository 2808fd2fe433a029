"""CPU tier: host-side pieces of bench.py.

A stored counter reading (profiles/traffic_*.json) is reported only while the
kernel's sources still hash to the reading's ``source_sha``.  The hash covers
code, not comments: a comment edit keeps the reading, any code edit drops it.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_blank_lines():
    src = "int a; // note\n\n/* block\n comment */ int b;   \n  // whole line\nint c;\n"
    assert bench._code_only(src) == "int a;\n int b;\nint c;"


def test_code_only_keeps_code_changes_visible():
    assert bench._code_only("x = 1; // one\n") != bench._code_only("x = 2; // one\n")
    assert bench._code_only("x = 1; // one\n") == bench._code_only("x = 1; // two\n")


def test_stored_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    kernel = "decode_bf16_kernel"
    d = {"source_sha": bench.kernel_source_sha(kernel), "bytes_per_launch": 123.0}
    (tmp_path / f"traffic_{kernel}.encdec_n1m.json").write_text(json.dumps(d))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic([kernel]) == 123.0
    d["source_sha"] = "0" * 16
    (tmp_path / f"traffic_{kernel}.encdec_n1m.json").write_text(json.dumps(d))
    assert bench.stored_traffic([kernel]) is None
