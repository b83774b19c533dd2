"""bench.py reports counter traffic only from a summary taken on the current decode
sources, for the workload and pool layout it covers (no GPU needed)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary(tmp_path, sha, layout="token", traffic=123456789):
    p = tmp_path / "traffic.md"
    p.write_text("# a summary\n\n| table | row |\n    an indented: line\n"
                 f"traffic_bytes_per_launch: {traffic}\npool_layout: {layout}\n"
                 f"kernel_sources_sha256: {sha}\n")
    return str(p)


def test_current_sources_give_the_value(tmp_path):
    p = _summary(tmp_path, bench.kernel_sources_sha256())
    assert bench.measured_traffic(p, "gqa_b64") == 123456789
    assert bench.measured_traffic(p, "gqa_b64", "token") == 123456789


def test_other_workload_layout_or_sources_give_none(tmp_path):
    p = _summary(tmp_path, bench.kernel_sources_sha256())
    assert bench.measured_traffic(p, "window_b32") is None
    assert bench.measured_traffic(p, "gqa_b64", "head") is None
    stale = _summary(tmp_path, "0" * 64)
    assert bench.measured_traffic(stale, "gqa_b64") is None
    assert bench.measured_traffic(str(tmp_path / "missing.md"), "gqa_b64") is None


def test_hash_covers_every_listed_source():
    assert all(os.path.exists(os.path.join(ROOT, f)) for f in bench.DECODE_SOURCES)
    assert len(bench.kernel_sources_sha256()) == 64


def test_committed_summary_parses():
    p = os.path.join(ROOT, "profiles", "decode_gqa_b64_hbm_traffic.md")
    v = bench.measured_traffic(p, "gqa_b64")
    assert v is None or v > 0
