"""Host-side logic of bench.py (no GPU): work counts, the whole-path lower bound, the gate
that keeps stale counter profiles out of the reported traffic, and the one-GPU guard."""
import json
import os
import subprocess
import sys
from itertools import combinations_with_replacement

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n,T", [(1, 1), (3, 2), (5, 7)])
def test_syrk_flops_counts_distinct_entries(n, T):
    # brute force: every entry (i, j), i <= j, of H = A^T A is a T-term dot product
    entries = sum(1 for _ in combinations_with_replacement(range(n), 2))
    assert bench.syrk_flops(n, T) == entries * 2 * T


def test_pipeline_lower_bound_terms():
    # 4096 x 4096 layer, 131072 tokens, block 128, 4 bits
    lb = bench.pipeline_lower_bound_ms(4096, 4096, 131072, 128, 4)
    # two SYRKs: 2 * 4096 * 4097 * 131072 = 4.399e12 flops at 2.5 PFLOP/s
    assert lb["syrk"] == pytest.approx(4.399e12 / 2.5e15 * 1e3, rel=1e-3)
    # feedback 4096 * 4096 * 3968 = 6.657e10 and factorization 2 * 4096^3 / 3 = 4.581e10
    # flops at 157.3 TFLOP/s
    assert lb["factor_and_feedback"] == pytest.approx((6.657e10 + 4.581e10) / 157.3e12 * 1e3,
                                                      rel=1e-3)
    # W, H_X, H_G read and written once in fp32 (3 * 2 * 64 MiB) and 16.8 M one-byte codes
    # packed to 8.4 MB, at 8 TB/s
    assert lb["hbm"] == pytest.approx((6 * 4096 * 4096 * 4 + 4096 * 4096 * 1.5) / 8e12 * 1e3,
                                      rel=1e-9)
    # the larger input side adds SYRK and factorization work
    wide = bench.pipeline_lower_bound_ms(4096, 11008, 131072, 128, 2)
    assert all(wide[k] > lb[k] for k in lb)


def _profile(tmp_path, src_text, recorded_hash, name="k_w1_hbm_traffic.json"):
    (tmp_path / "profiles").mkdir(exist_ok=True)
    src = tmp_path / "k.hip"
    src.write_text(src_text)
    (tmp_path / "profiles" / name).write_text(json.dumps(
        {"kernel_source_sha256_16": recorded_hash, "hbm_bytes_per_launch": 123456789}))
    return str(src)


def test_traffic_taken_only_from_a_profile_of_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = _profile(tmp_path, "kernel v1", "0" * 16)
    current = bench.source_hash(src)
    _profile(tmp_path, "kernel v1", current)
    assert bench.traffic_from_profile(src, "k", "w1") == 123456789
    # another workload's counters are not this one's
    assert bench.traffic_from_profile(src, "k", "w2") is None
    # the kernel changed after the counters were taken: no traffic figure
    with open(src, "w") as f:
        f.write("kernel v2")
    assert bench.traffic_from_profile(src, "k", "w1") is None
    # no profile at all
    assert bench.traffic_from_profile(src, "missing", "w1") is None


def test_committed_profiles_name_their_kernel_source():
    for name in ("syrk_dma_kernel_c2_hbm_traffic.json", "qform_kernel_c2_hbm_traffic.json"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            d = json.load(f)
        assert len(d["kernel_source_sha256_16"]) == 16
        assert d["hbm_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
