"""Host logic of bench.py (CPU only): the kernel-source hash that keeps the
committed traffic counters tied to the code they were taken on, the binding
roof, and the traffic lookup."""

import json
import os

import pytest

import bench


@pytest.fixture
def fake_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a kernel\nint f(int x) {\n  return x + 1;  /* one */\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    return src


def test_hash_ignores_comments_and_whitespace(fake_sources):
    h0 = bench.kernel_source_hash()
    fake_sources.write_text("/* a kernel,\n   reworded */\nint f(int x)\n{ return x + 1; }\n")
    assert bench.kernel_source_hash() == h0


def test_hash_follows_code(fake_sources):
    h0 = bench.kernel_source_hash()
    fake_sources.write_text("// a kernel\nint f(int x) {\n  return x + 2;  /* one */\n}\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_only_for_the_same_code(fake_sources, tmp_path):
    (tmp_path / "profiles").mkdir()
    entry = {"entries": {"w/T=8/k_up": {"bytes_per_launch": 123.0}}}
    path = tmp_path / "profiles" / "hbm_traffic.json"
    path.write_text(json.dumps(dict(entry, kernel_source_hash=bench.kernel_source_hash())))
    assert bench.load_traffic("w", 8, "k_up") == 123.0
    assert bench.load_traffic("w", 16, "k_up") is None
    path.write_text(json.dumps(dict(entry, kernel_source_hash="0" * 16)))
    assert bench.load_traffic("w", 8, "k_up") is None


def test_binding_roof():
    # 1 TFLOP and 1 GB: 200 us at the 5.0 PFLOP/s e4m3 peak against 125 us at
    # 8 TB/s, so the MFMA roof binds; measured 400 us -> half of it
    bound, t, frac = bench.roof(1e12, 1e9, 400.0, "fp8_blockwise")
    assert bound == "mfma" and t == pytest.approx(200.0) and frac == pytest.approx(0.5)
    bound, t, frac = bench.roof(1e11, 4e9, 1000.0, "fp8_blockwise")
    assert bound == "hbm" and t == pytest.approx(500.0) and frac == pytest.approx(0.5)

