"""Host logic of bench.py and of the workload table (CPU only).

The expected sizes are those of the one-GPU shares used to evaluate LRMoE
("LRMoE: Trimming Backward Work in Memory-Bound MoE Training", section "What
the measurements show": Qwen3-30B-A3B and GLM4.5-106B-A12B shapes, C20/C30
quotas, the 20x batch-pressure share under a fixed token-buffer budget),
written out from the shapes by hand: routed pairs, kept pairs, bytes the
score / select / compaction steps must move and the matrix work of the two
gradients.
"""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

import bench
from oracle import lrmoe_oracle as O
from pruned_expert_backward_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# config: (P, E, d_out, d_in, kept pairs M, largest and smallest expert)
SHARES = {
    1: (32768, 16, 2048, 768, 26210, 11970, 430),
    2: (32768, 16, 2048, 768, 22930, 16584, 196),
    3: (32768, 16, 4096, 1408, 26210, 11970, 430),
    4: (655360, 16, 4096, 1408, 63108, 286057, 5898),
}


@pytest.mark.parametrize("c", sorted(SHARES))
def test_routing_and_kept_pairs(c):
    P, E, d_out, d_in, M, n_max, n_min = SHARES[c]
    spec = W.CONFIGS[c]
    assert (spec["P"], spec["E"], spec["d_out"], spec["d_in"]) == (P, E, d_out, d_in)
    counts = W.zipf_counts(P, E, spec["zipf"], 1000 + c)
    assert int(counts.sum()) == P
    assert (int(counts.max()), int(counts.min())) == (n_max, n_min)
    q = O.plan_quota(counts, spec["policy"])
    assert int(np.sum(q)) == M


def _share(c):
    P, E, d_out, d_in, M, _, _ = SHARES[c]
    return types.SimpleNamespace(P=P, E=E, d_out=d_out, d_in=d_in, dtype="bf16"), M


@pytest.mark.parametrize("c,score_mb,compact_mb,zero_mb,dw_gflop", [
    # bf16 rows: score reads g and phi (2 bytes each) plus alpha, writes R
    (1, 184.8, 295.5, 20.1, 82.5),
    (3, 361.0, 577.4, 36.9, 302),
    (4, 7219.4, 1390.1, 3335.6, 728),
])
def test_algorithmic_work(c, score_mb, compact_mb, zero_mb, dw_gflop):
    p, M = _share(c)
    # score + select (R read, keep flag written: 5 bytes a pair) + compaction
    # (kept rows read and written, alpha and perm) + zero rows of dropped pairs
    want = (score_mb + compact_mb + zero_mb) * 1e6 + 5 * p.P
    # (each figure given to 0.1 MB)
    assert bench.algorithmic_bytes(p, M) == pytest.approx(want, abs=1.5e5)
    # dW and dphi: 2 * M * d_out * d_in each (dW given to three digits)
    assert bench.gemm_flops(p, M) == pytest.approx(2 * dw_gflop * 1e9, rel=2e-3)
    # gradient-only score rules read g only; caller-given scores read nothing
    g_only = p.P * (2 * p.d_out + 4)
    full = p.P * (2 * (p.d_out + p.d_in) + 8)
    assert (bench.algorithmic_bytes(p, M) - bench.algorithmic_bytes(p, M, "grad-sqnorm")
            == full - g_only)
    assert bench.algorithmic_bytes(p, M) - bench.algorithmic_bytes(p, M, "random") == full


def test_gemm_floor_bytes():
    p, M = _share(4)
    operands = M * 2 * (p.d_out + p.d_in) + p.E * p.d_out * p.d_in * 2   # g_c, phi_c, W
    outputs = p.E * p.d_out * p.d_in * 4 + M * p.d_in * 4              # dW, kept dphi rows
    assert bench.gemm_floor_bytes(p, M) == operands + outputs


def _summary(path, **kv):
    base = dict(workload="glm45-106b-a12b-20x-budget", leg="down", dw_mode="f16",
                kernel="grouped_backward_kernel<1, 1, 1, 1, 0, 3>",
                kernel_sources_sha256=bench.gemm_sources_sha256(),
                gemm_fetch_kib="1000.0", gemm_write_kib="3000.0", copy_bytes="1073741824",
                copy_fetch_kib="524288.0", copy_write_kib="1048576.0",
                mfma_busy_frac="0.4")
    base.update(kv)
    with open(path, "w") as f:
        f.write("# comment lines are skipped = even with an equals sign\n")
        for k, v in base.items():
            if v is not None:
                f.write(f"{k} = {v}\n")


def test_read_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS_GLOB", str(tmp_path / "*.counters.txt"))
    _summary(tmp_path / "a.counters.txt")
    traffic, busy = bench.read_counters("glm45-106b-a12b-20x-budget", "f16")
    # FETCH scaled by 2 (the copy read 2^30 bytes as 2^19 KiB), WRITE by 1
    assert traffic == pytest.approx(1000.0 * 2048 + 3000.0 * 1024)
    assert busy == pytest.approx(0.4)
    # another workload, dW mode or leg: nothing
    assert bench.read_counters("qwen3-30b-a3b-down-c20", "f16") == (None, None)
    assert bench.read_counters("glm45-106b-a12b-20x-budget", "exact") == (None, None)
    assert bench.read_counters("glm45-106b-a12b-20x-budget", "f16", "gate_up") == (None, None)


def test_read_counters_skips_stale_or_broken_summaries(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS_GLOB", str(tmp_path / "*.counters.txt"))
    _summary(tmp_path / "a.counters.txt", kernel_sources_sha256="0" * 64)   # other sources
    _summary(tmp_path / "b.counters.txt", gemm_write_kib=None)              # key missing
    _summary(tmp_path / "c.counters.txt", copy_fetch_kib="0")               # no calibration
    assert bench.read_counters("glm45-106b-a12b-20x-budget", "f16") == (None, None)
    _summary(tmp_path / "d.counters.txt", mfma_busy_frac=None)
    traffic, busy = bench.read_counters("glm45-106b-a12b-20x-budget", "f16")
    assert traffic is not None and busy is None


def test_committed_profiles_parse():
    """Every committed GEMM counter summary carries what bench.py reads."""
    import glob
    paths = sorted(glob.glob(os.path.join(ROOT, bench.COUNTERS_GLOB)))
    assert paths
    names = {W.CONFIGS[c]["name"] for c in SHARES}
    seen = set()
    for path in paths:
        kv = {}
        for line in open(path):
            if line.strip() and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        seen.add(kv["workload"])
        assert len(kv["kernel_sources_sha256"]) == 64
        for k in ("gemm_fetch_kib", "gemm_write_kib", "copy_fetch_kib", "copy_write_kib"):
            assert float(kv[k]) > 0
        assert 0.0 < float(kv["mfma_busy_frac"]) < 1.0
    assert seen == names


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
