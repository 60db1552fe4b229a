"""Host-side pieces of bench.py: the one-GPU refusal and the counter-traffic
reading (copy-calibrated FETCH_SIZE + WRITE_SIZE, null once the decode kernel
sources change)."""
import json
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _summary(tmp_path, digest, fetch=1000.0, write=10.0, copy_fetch=500.0, copy_write=1000.0):
    rec = {"decode_source_sha256": digest, "decode_fetch_kib": fetch, "decode_write_kib": write,
           "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write, "copy_bytes": 1000 * 1024}
    p = tmp_path / "counters.md"
    p.write_text("# summary\n\n```json\n" + json.dumps(rec) + "\n```\n")
    return str(p)


def test_traffic_is_scaled_by_the_copy(tmp_path, monkeypatch):
    # copy moved 1000 KiB each way; FETCH read 500 (x2), WRITE read 1000 (x1)
    monkeypatch.setattr(bench, "COUNTER_SUMMARY", _summary(tmp_path, bench.decode_source_digest()))
    traffic, why = bench.counter_traffic()
    assert why is None
    assert traffic == pytest.approx((1000.0 * 2 + 10.0) * 1024)


def test_traffic_null_once_sources_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTER_SUMMARY", _summary(tmp_path, "0" * 64))
    traffic, why = bench.counter_traffic()
    assert traffic is None and "changed" in why


def test_committed_summary_parses():
    traffic, why = bench.counter_traffic()
    if why is not None:
        pytest.skip(why)
    # the decode launch reads K^ and V^ once: counters must not fall below that
    assert traffic >= 2 * 131072 * 8 * 128 * 2


def test_committed_prefill_counters_parse():
    busy, why = bench.prefill_mfma_busy()
    if why is not None:
        pytest.skip(why)
    assert 0.3 < busy <= 1.0


def test_prefill_busy_null_once_sources_change(tmp_path, monkeypatch):
    p = tmp_path / "pf.md"
    p.write_text('```json\n{"prefill_source_sha256": "' + "0" * 64 + '", "mfma_busy_cycles": 1, '
                 '"gui_active_cycles": 8, "simds": 1, "xcds": 8}\n```\n')
    monkeypatch.setattr(bench, "PREFILL_COUNTER_SUMMARY", str(p))
    busy, why = bench.prefill_mfma_busy()
    assert busy is None and "changed" in why
