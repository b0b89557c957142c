"""Host-side helpers of bench.py (no GPU): the committed counter summary is
read back only while the attention sources match the hash it was taken on."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_profiled_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    b = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    md = prof / "attn_mfma_kernel__w__hbm_traffic.md"
    h = b.attn_source_hash()
    md.write_text("# summary\n\n- kernel_source_sha256: `%s`\n- traffic_bytes_per_launch: `12345`\n" % h)
    # the hash is of the real sources; only the summary lives in tmp_path
    monkeypatch.setattr(b, "attn_source_hash", lambda: h)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.profiled_traffic("w") == 12345.0
    md.write_text("- kernel_source_sha256: `00`\n- traffic_bytes_per_launch: `12345`\n")
    assert b.profiled_traffic("w") is None
    assert b.profiled_traffic("absent") is None


def test_committed_summary_parses():
    b = _bench()
    path = os.path.join(ROOT, "profiles", "attn_mfma_kernel__sdxl_bf16__hbm_traffic.md")
    if not os.path.exists(path):
        pytest.skip("no committed counter summary")
    text = open(path).read()
    assert "kernel_source_sha256" in text and "traffic_bytes_per_launch" in text
    # parses to a number whenever the sources still match
    val = b.profiled_traffic("sdxl_bf16")
    assert val is None or val > 0
