"""Host-side logic of bench.py (no GPU): the measured HBM traffic it reports.

The attention pass's traffic comes from rocprofv3 counter runs on one
workload and one version of the attention source; any other workload, or a
changed source, must report null rather than a stale figure.
"""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_only_for_the_counted_workload():
    b = _bench()
    t = b.ATTN_TRAFFIC
    counted = t["workload"]
    assert b.attn_traffic("ragged_b64_l1k_32k") is None
    assert b.attn_traffic("mtp_b128_sq2_l2k_16k") is None
    if t["src_sha256"] == b.attn_source_hash():
        got = b.attn_traffic(counted)
        want = (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0
        assert got == want
        # at least the algorithmic bytes: 131072 cached tokens x 1152 B
        assert got >= 131072 * 1152
    else:
        assert b.attn_traffic(counted) is None


def test_traffic_null_after_a_source_change(monkeypatch):
    b = _bench()
    monkeypatch.setitem(b.ATTN_TRAFFIC, "src_sha256", "0" * 64)
    assert b.attn_traffic(b.ATTN_TRAFFIC["workload"]) is None


def test_counted_workload_is_the_default_bench_workload():
    from mla_latent_kv_amd import synth
    b = _bench()
    assert b.ATTN_TRAFFIC["workload"] == synth.CONFIGS[1].name
