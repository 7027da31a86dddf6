"""Host-side checks of bench.py: the one-GPU guard, the algorithmic FLOP
counts it divides by (against brute-force enumeration of the pairs they
count), and the source-keyed HBM traffic lookup. No GPU needed."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ssa_inputs import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("name", ["tiny_f32", "mha_4k", "gqa_32k_sweep", "paper_16k_b16"])
def test_prefill_flops_count_causal_pairs(name):
    cfg = CONFIGS[name]
    nkb = cfg.N // cfg.block
    pairs = sum(1 for qb in range(nkb) for kb in range(nkb) if kb <= qb)
    # QK^T and PV: 2 D FLOPs each per (query row, key) of a block pair
    expect = pairs * cfg.block * cfg.block * (2 * cfg.D + 2 * cfg.D) * cfg.B * cfg.Hq
    assert bench.prefill_flops(cfg) == expect


def test_prefill_flops_32k_value():
    # 512 query blocks, 131328 causal block pairs, 32 heads, D 128
    assert bench.prefill_flops(CONFIGS["gqa_32k_sweep"]) == pytest.approx(8.813e12, rel=1e-3)


@pytest.mark.parametrize("name,n_sink,n_local", [("tiny_f32", 1, 1), ("mha_4k", 1, 1),
                                                  ("tiny_f32", 0, 2), ("tiny_f32", 2, 0)])
def test_token_select_flops_enumerates_candidates(name, n_sink, n_local):
    cfg = CONFIGS[name].with_sizes(n_sink=n_sink, n_local=n_local)
    nkb = cfg.N // cfg.block
    cand = 0
    for row in range(cfg.N):
        qb = row // cfg.block
        for kb in range(qb + 1):
            forced = kb < n_sink or kb > qb - n_local
            cand += 0 if forced else 1
    assert bench.token_select_flops(cfg, cfg.budget) == 2.0 * cfg.D * cand * cfg.B * cfg.Hq
    assert nkb >= 1


def test_sparse_flops_counts_selected_pairs():
    cfg = CONFIGS["mha_4k"]
    cnt = np.array([[[3, 5, 16]], [[1, 0, 2]]])
    assert bench.sparse_flops(cfg, cnt) == 4.0 * cfg.D * cfg.block * cfg.block * 27


def test_traffic_is_keyed_by_source(tmp_path, monkeypatch):
    f = tmp_path / "k.hip"
    f.write_bytes(b"kernel source")
    monkeypatch.setattr(bench, "PREFILL_SRCS", [str(f)])
    sha = bench.prefill_source_sha()
    monkeypatch.setattr(bench, "PREFILL_TRAFFIC", {sha: 1234})
    assert bench.prefill_traffic() == 1234
    f.write_bytes(b"kernel source, edited")
    assert bench.prefill_traffic() is None
    monkeypatch.setattr(bench, "PREFILL_SRCS", [str(tmp_path / "missing.hip")])
    assert bench.prefill_traffic() is None
