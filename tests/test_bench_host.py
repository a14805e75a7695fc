"""Host logic of bench.py: the algorithmic byte and flop counts behind the reported
rooflines, and the rule that a counter summary is only reported while it matches the
sources it was taken on.

The expected counts are worked out here from the workload definitions (configurations 2
to 4 of the benchmark: the Llama-3-8B-shaped layer, the token-dropping draft and the
Qwen3-30B-A3B-shaped layer), term by term, independently of bench.py's formulas.
"""
import importlib.util
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    spec = importlib.util.spec_from_file_location("bench_host_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _qo_bytes(w):
    # one bf16 query row in, one bf16 output row out per q-head
    return 2 * w.B * w.Hq * w.d * 2


def test_quant_decode_bytes_llama8b(bench):
    w = bench.workload("llama8b")
    bh = 8 * 8
    codes = bh * 32768 * 128 * (4 + 4) // 8          # 4-bit K and V codes
    k_params = bh * (32768 // 64) * 128 * 2 * 2       # per-channel K scale + zero per 64-token group, bf16
    v_params = bh * 32768 * (128 // 64) * 2 * 2       # per-token V scale + zero per 64-channel group, bf16
    assert codes + k_params + v_params == 301_989_888
    assert bench.decode_bytes(w, 32768, 0) - _qo_bytes(w) == 301_989_888


def test_quant_decode_bytes_qwen30b(bench):
    w = bench.workload("qwen30b")
    bh = 16 * 4
    codes = bh * 65536 * 128 * (4 + 3) // 8
    k_params = bh * (65536 // 32) * 128 * 2 * 2
    v_params = bh * 65536 * (128 // 32) * 2 * 2
    assert codes + k_params + v_params == 603_979_776
    assert bench.decode_bytes(w, 65536, 0) - _qo_bytes(w) == 603_979_776


def test_kept_row_decode_bytes_drop(bench):
    w = bench.workload("drop")
    kept = 131072 // 4
    assert bench.decode_bytes(w, kept, 0) - _qo_bytes(w) == 4 * 8 * kept * 128 * 2 * 2 == 536_870_912


def test_tail_rows_counted_as_bf16_k_and_v(bench):
    w = bench.workload("llama8b")
    assert bench.decode_bytes(w, 32768, 40) - bench.decode_bytes(w, 32768, 0) == 8 * 8 * 40 * 128 * 2 * 2


# the verify work of the three layers to one decimal: 137.5, 343.6 and 687.4 GFLOP
@pytest.mark.parametrize("name, n, gflop", [("llama8b", 32768, 137.5), ("drop", 131072, 343.6),
                                            ("qwen30b", 65536, 687.4)])
def test_verify_flops(bench, name, n, gflop):
    # QK^T and PV: 2 * 2 * d flops per (q-head row, visible key); window row i sees n + i + 1 keys
    w = bench.workload(name)
    keys = sum(n + i + 1 for i in range(w.k))
    assert 4 * w.B * w.Hq * w.d * keys == bench.verify_flops(w, n)
    assert abs(bench.verify_flops(w, n) / 1e9 - gflop) < 0.1


def test_verify_bytes_llama8b(bench):
    w = bench.workload("llama8b")
    kv = 8 * 8 * (32768 + 32) * 128 * 2 * 2
    q_o = 2 * 8 * 32 * 32 * 128 * 2
    assert bench.verify_bytes(w, 32768) == kv + q_o


def _recorded_hash(bench, name):
    with open(os.path.join(bench.ROOT, "profiles", bench.TRAFFIC[name][0])) as fh:
        for line in fh:
            if line.startswith("# source_sha256:"):
                return line.split(":", 1)[1].strip()
    return None


def test_traffic_reported_only_for_matching_sources(bench, monkeypatch):
    # sources hashed as the summary recorded: the figure is reported
    for name in bench.TRAFFIC:
        rec = _recorded_hash(bench, name)
        assert rec, name
        monkeypatch.setattr(bench, "source_hash", lambda files, rec=rec: rec)
        t = bench.measured_traffic(name)
        assert t is not None and t > 0, name
    assert bench.measured_traffic("no_such_workload") is None
    # any other sources: not reported
    monkeypatch.setattr(bench, "source_hash", lambda files: "0" * 16)
    for name in bench.TRAFFIC:
        assert bench.measured_traffic(name) is None, name
