"""Host logic of bench.py (no GPU): the single-GPU guard, the algorithmic byte counts the roofline divides by,
and the rule that a counter summary taken on other kernel sources is not reported."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import tpa_inputs as ti  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_bytes_by_hand():
    """The ragged workload: 128 sequences, h=32, d_h=128, R_K=R_V=4, bf16.  Per cached token the cache holds
    (4 + 4) x (32 + 128) bf16 factors = 2560 B; per sequence the decode also reads its bf16 query (32 x 128 x 2 B)
    and writes its fp32 output (32 x 128 x 4 B); a fused step also reads the new token's 2560 B of factors and
    writes its 2560 B record."""
    w = ti.get("ragged")
    lens = ti.decode_lengths(w)
    assert len(lens) == 128 and int(np.sum(lens)) == 2_265_395
    decode = 2_265_395 * 2560 + 128 * (32 * 128 * 2 + 32 * 128 * 4)
    assert bench.decode_bytes(w, lens) == decode == 5_802_556_928
    assert bench.step_bytes(w, lens) == decode + 128 * (2560 + 2560) == 5_803_212_288


def test_e4m3_bytes_by_hand():
    """An E4M3 cache stores one byte per factor element: 1280 B per token at the ragged workload's shape; the
    query, output and the new token's factors keep their bf16/fp32 sizes, the record is 1280 B."""
    w = ti.get("ragged")
    lens = ti.decode_lengths(w)
    decode = 2_265_395 * 1280 + 128 * (32 * 128 * 2 + 32 * 128 * 4)
    assert bench.decode_bytes(w, lens, cache_es=1) == decode
    assert bench.step_bytes(w, lens, cache_es=1) == decode + 128 * (2560 + 1280)


def test_counter_summary_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    current = bench.source_hash(bench.PREFILL_SOURCES)
    (tmp_path / "match.json").write_text(json.dumps({"source_hash": current, "mfma_busy_frac": 0.3}))
    (tmp_path / "stale.json").write_text(json.dumps({"source_hash": "0" * 16, "mfma_busy_frac": 0.3}))
    (tmp_path / "broken.json").write_text("{not json")
    assert bench.profile_record("match", bench.PREFILL_SOURCES)["mfma_busy_frac"] == 0.3
    assert bench.profile_record("stale", bench.PREFILL_SOURCES) is None
    assert bench.profile_record("broken", bench.PREFILL_SOURCES) is None
    assert bench.profile_record("missing", bench.PREFILL_SOURCES) is None


def test_committed_summaries_match_the_committed_kernels():
    """The summaries under profiles/ that the benchmark line reports were taken on the kernel sources in the
    tree (otherwise the line carries null traffic and busy fraction)."""
    assert bench.profile_record("mfma_busy_prefill_b8_ctx2048_chunk512", bench.PREFILL_SOURCES) is not None
    for name in bench.DECODE_WORKLOADS:
        w = ti.get(name)
        assert bench.profile_record("hbm_bytes_" + w.name, bench.DECODE_SOURCES) is not None, w.name
