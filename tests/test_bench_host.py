"""Host-side checks of bench.py's counter lookups (no GPU): the HBM traffic it
reports comes from committed rocprofv3 counters only while those were taken on
the current kernel source and workload."""

import json

import bench


def _write(path, rec):
    path.write_text(json.dumps(rec))
    return str(path)


def test_verify_traffic_needs_current_digest_and_workload(tmp_path, monkeypatch):
    rec = {"workload": "prod", "kernel_source_sha256_16": bench.kernel_source_digest(), "hbm_bytes_per_launch": 123}
    monkeypatch.setattr(bench, "COUNTERS_FILE", _write(tmp_path / "c.json", rec))
    assert bench.measured_traffic("prod") == 123
    assert bench.measured_traffic("gqa8") is None
    rec["kernel_source_sha256_16"] = "0" * 16
    monkeypatch.setattr(bench, "COUNTERS_FILE", _write(tmp_path / "d.json", rec))
    assert bench.measured_traffic("prod") is None
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("prod") is None


def test_prefill_traffic_per_mask(tmp_path, monkeypatch):
    rec = {"workload": "prefill_12k", "prefill_source_sha256_16": bench.prefill_source_digest(),
           "hbm_bytes_per_launch": {"non_causal": 10, "causal": 20}}
    monkeypatch.setattr(bench, "PREFILL_COUNTERS_FILE", _write(tmp_path / "p.json", rec))
    assert bench.prefill_traffic("prefill_12k", False) == 10
    assert bench.prefill_traffic("prefill_12k", True) == 20
    assert bench.prefill_traffic("prefill_small", False) is None
    rec["prefill_source_sha256_16"] = bench.kernel_source_digest()   # another kernel's digest
    monkeypatch.setattr(bench, "PREFILL_COUNTERS_FILE", _write(tmp_path / "q.json", rec))
    assert bench.prefill_traffic("prefill_12k", False) is None


def test_digests_ignore_comments(tmp_path, monkeypatch):
    """A comment-only change keeps a digest; a code change moves it."""
    src = tmp_path / "paged_fp8_kv_split_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "a.hip").write_text("int f() { return 1; }  // one\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench._code_digest(("a.hip",))
    (src / "a.hip").write_text("// lead\nint f() { return 1; }  // two\n\n")
    assert bench._code_digest(("a.hip",)) == d0
    (src / "a.hip").write_text("int f() { return 2; }\n")
    assert bench._code_digest(("a.hip",)) != d0
