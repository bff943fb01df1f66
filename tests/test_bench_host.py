"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the per-step
FLOP / byte models against the layer's FLOP count, and the staleness check of
the committed counter summaries."""
import glob
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import lmoe_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", sorted(S.CONFIGS))
def test_step_flops_add_up_to_the_layer(name):
    """The timed steps together perform exactly the layer's algorithmic FLOPs."""
    cfg = S.CONFIGS[name]
    counts = np.full(cfg.n_routed, cfg.pairs // cfg.n_routed, dtype=np.int64)
    models = bench.step_models(cfg, counts)
    assert sum(f for f, _ in models.values()) == pytest.approx(cfg.flops(), rel=1e-12)


def test_routed_bytes_count_only_experts_with_pairs():
    cfg = S.CONFIGS["k3full_n64"]
    R, l, f = cfg.n_routed, cfg.d_latent, cfg.ff_routed
    all_used = bench.step_models(cfg, np.ones(R, dtype=np.int64))
    some = np.zeros(R, dtype=np.int64)
    some[:10] = 1
    few_used = bench.step_models(cfg, some)
    es = 2
    # each expert without pairs saves its gate and up (and down) weights
    assert all_used["routed_gateup"][1] - few_used["routed_gateup"][1] == (R - 10) * 2 * f * l * es
    assert all_used["routed_down"][1] - few_used["routed_down"][1] == (R - 10) * l * f * es


def test_kernel_hash_covers_every_kernel_source():
    csrc = os.path.join(ROOT, "mixture_experts_ffn_sigmoid_amd", "csrc")
    files = {os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "*.hip"))}
    assert files <= set(bench.KERNEL_SOURCES), files - set(bench.KERNEL_SOURCES)


def test_traffic_summary_is_ignored_when_kernels_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_routed_gateup_w.txt").write_text(
        "# counters\nsource_hash: 0123456789abcdef\ntraffic_bytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.measured_traffic("routed_gateup", "w") == 1234.0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.measured_traffic("routed_gateup", "w") is None
    assert bench.measured_traffic("routed_down", "w") is None
