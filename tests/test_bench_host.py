"""Host-side pieces of bench.py: the algorithmic counts, the traffic table and
the host report (no GPU needed)."""

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_alg_counts_long_64k(bench):
    # 6 d_k d_v + 2 C (3 d_k + 2 d_v) = 118,784 flop and 2 (2 d_k + d_v) + 2 d_v + 8
    # = 1,032 bytes per token and head, plus the fp32 final state once per head
    flops, byts = bench.alg_counts(1, 65536, 16, 128, 128)
    assert flops == 65536 * 16 * 118784
    assert byts == 65536 * 16 * 1032 + 16 * 128 * 128 * 4
    _, with_h0 = bench.alg_counts(1, 65536, 16, 128, 128, h0=True)
    assert with_h0 == byts + 16 * 128 * 128 * 4


def test_traffic_table_sources_exist(bench):
    for entry in bench.TRAFFIC_KIB.values():
        assert len(bench.source_hash(entry["sources"])) == 16
        assert entry["fetch"] > 0 and entry["write"] > 0


def test_traffic_only_for_long_64k(bench):
    assert bench.measured_traffic("chunk", "train_8k") is None


def test_host_info(bench):
    info = bench.host_info()
    assert info["nproc"] == os.cpu_count()
    assert isinstance(info["cpu_model"], str) and info["cpu_model"]
