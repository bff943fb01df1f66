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
    assert sum(f for f, _, _ in models.values()) == pytest.approx(cfg.flops(), rel=1e-12)


def test_routed_bytes_count_only_experts_with_pairs():
    cfg = S.CONFIGS["k3full_n64"]
    R, l, f = cfg.n_routed, cfg.d_latent, cfg.ff_routed
    all_used = bench.step_models(cfg, np.ones(R, dtype=np.int64))
    some = np.zeros(R, dtype=np.int64)
    some[:10] = 1
    few_used = bench.step_models(cfg, some)
    es = 2
    # each expert without pairs saves its gate and up (and down) weights
    for j in (1, 2):  # algorithmic and design bytes
        assert all_used["routed_gateup"][j] - few_used["routed_gateup"][j] == (R - 10) * 2 * f * l * es
        assert all_used["routed_down"][j] - few_used["routed_down"][j] == (R - 10) * l * f * es
    some_layer = bench.layer_algorithmic_bytes(cfg, some)
    assert bench.layer_algorithmic_bytes(cfg, np.ones(R, dtype=np.int64)) - some_layer == (R - 10) * 3 * f * l * es


def test_algorithmic_bytes_follow_the_weights_once_model():
    """Routed gate/up: the touched W_g and W_u plus z read once; the per-pair
    gather and h are design bytes (fp16 intermediates with bf16 storage)."""
    cfg = S.CONFIGS["k3full_n8192"]
    N, l, R, k, f = cfg.n_tokens, cfg.d_latent, cfg.n_routed, cfg.top_k, cfg.ff_routed
    m = bench.step_models(cfg, np.full(R, N * k // R))
    assert m["routed_gateup"][1] == 2 * (2 * R * f * l) + 2 * N * l
    assert m["routed_gateup"][2] == 2 * (2 * R * f * l) + 2 * (N * k * l + N * k * f)
    assert m["routed_down"][1] == 2 * R * l * f
    assert m["routed_down"][2] == 2 * R * l * f + 2 * (N * k * f + N * k * l)
    assert m["combine_rmsnorm"][1] == 0 and m["combine_rmsnorm"][2] == 2 * (N * k * l + N * l)


# Per-step device times (ms) measured by bench.py's HIP events on an MI355X
# (full-K3 prefill and few-token layers, the kernels of the first measured build).
RECORDED_STEP_MS = {
    "k3full_n8192": {"latent_gemm": 0.3736, "router": 0.1825, "dispatch": 0.1130, "shared_gateup": 3.5484,
                     "routed_gateup": 5.9159, "routed_down": 3.5681, "combine_rmsnorm": 0.2051, "merge_gemm": 2.8372},
    "k3full_n64": {"latent_gemm": 0.0241, "router": 0.0424, "dispatch": 0.0535, "shared_gateup": 0.1325,
                   "routed_gateup": 2.9366, "routed_down": 1.5457, "combine_rmsnorm": 0.0165, "merge_gemm": 0.0843},
}


@pytest.mark.parametrize("name", sorted(RECORDED_STEP_MS))
def test_no_step_exceeds_peak_for_recorded_times(name):
    """A byte or FLOP model that claims more than the hardware can do is
    wrong: for recorded step times, every step's algorithmic and design
    bytes per second stay below the HBM peak, its FLOP/s below the MFMA peak."""
    cfg = S.CONFIGS[name]
    counts = np.full(cfg.n_routed, max(1, cfg.pairs // cfg.n_routed))
    if name == "k3full_n64":  # about 610 experts receive the 1024 pairs
        counts[610:] = 0
    models = bench.step_models(cfg, counts)
    peak_tf = bench.PEAK_MFMA_TFLOPS[cfg.dtype]
    for step, ms in RECORDED_STEP_MS[name].items():
        fl, alg, design = models[step]
        t = ms / 1e3
        assert fl / t / 1e12 < peak_tf, (step, fl / t / 1e12)
        assert alg / t / 1e9 < bench.PEAK_HBM_GBS, (step, alg / t / 1e9)
        assert design / t / 1e9 < bench.PEAK_HBM_GBS, (step, design / t / 1e9)


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
