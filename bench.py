"""Throughput of the MI355X Stable LatentMoE forward on one GPU.

One step = one whole-layer forward (latent GEMM, routing, dispatch, shared and
routed SiTU experts, RMSNorm merge) over one batch of seeded synthetic input
already resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lmoe_synth as S  # noqa: E402

METRIC = "LatentMoE fwd tokens/s + TFLOP/s at 1 MI355X; % of bf16 MFMA / HBM roofline"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense matrix peaks (fp16 == bf16)
PEAK_HBM_GBS = 8000.0


def step_models(cfg, counts):
    """Per timed step: (algorithmic FLOPs, algorithmic HBM bytes, design HBM bytes).

    FLOPs: 2 per multiply-add; the routed work counts the N*k token-expert
    pairs (no padding).  Algorithmic bytes: the weights the step needs, each
    read once (routed experts: only those with pairs), plus the layer's input
    x (read by each step that uses it) and output y at the storage width, the
    latent z once at the intermediate width (written by the latent step, read
    by the routed gate/up), and the router's ids and p.  Design bytes: what
    this implementation moves by design on top of that: the per-pair gather
    of z rows, the routed hidden h, the p-weighted slot rows, the shared
    hidden, RMSNorm(u) and the router logits (fp16 intermediates with bf16
    storage, fp32 with fp32 storage).  Returns {step: (flops, alg, design)}."""
    N, d, l, R, k = cfg.n_tokens, cfg.d_model, cfg.d_latent, cfg.n_routed, cfg.top_k
    fr, fs, ns = cfg.ff_routed, cfg.ff_shared, cfg.n_shared
    es = 2 if cfg.dtype == "bf16" else 4  # storage
    ei = es  # intermediates: fp16 (bf16 storage) or fp32
    P = N * k
    U = int((counts > 0).sum())
    w_gu, w_o = es * 2 * U * fr * l, es * U * l * fr
    return {
        "latent_gemm": (2.0 * N * d * l, es * (N * d + l * d) + ei * N * l, es * (N * d + l * d) + ei * N * l),
        "router": (2.0 * N * d * R, es * (N * d + R * d) + 8 * N * k, es * (N * d + R * d) + 8 * N * k + 8 * N * R),
        "dispatch": (0.0, 8 * P, 8 * P + 8 * R),
        "shared_gateup": (4.0 * N * d * fs * ns, es * (N * d + 2 * ns * fs * d),
                          es * (N * d + 2 * ns * fs * d) + ei * N * ns * fs),
        "routed_gateup": (4.0 * P * l * fr, w_gu + ei * N * l, w_gu + ei * (P * l + P * fr)),
        "routed_down": (2.0 * P * fr * l, w_o, w_o + ei * (P * fr + P * l)),
        "combine_rmsnorm": (0.0, 0, ei * (P * l + N * l)),
        "merge_gemm": (2.0 * N * (ns * fs + l) * d, es * (d * (ns * fs + l) + N * d),
                       es * (d * (ns * fs + l) + N * d) + ei * N * (ns * fs + l)),
    }


def layer_algorithmic_bytes(cfg, counts) -> float:
    """The whole layer's algorithmic HBM bytes: every needed weight once
    (routed experts with pairs only), x read once and y written once."""
    N, d, l, R = cfg.n_tokens, cfg.d_model, cfg.d_latent, cfg.n_routed
    fr, fs, ns = cfg.ff_routed, cfg.ff_shared, cfg.n_shared
    es = 2 if cfg.dtype == "bf16" else 4
    U = int((counts > 0).sum())
    weights = l * d + R * d + 3 * U * fr * l + 3 * ns * fs * d + d * l
    return float(es * (weights + 2 * N * d))


def host_cpu() -> dict:
    """Cores this process may run on (sched_getaffinity) and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(cfg, n_sample: int, threads: int | None = None, device_experts: bool = False):
    """The oracle (test infrastructure, untuned) on the first n_sample tokens of
    the workload, on this host's cores (BLAS threads = `threads`, default all
    cores of the affinity mask).  The routed experts the sample needs are
    generated beforehand on the host, or, with device_experts, copied as the
    oracle asks for them from the device copy of the seeded weights (cast to
    fp64 on the device, which is exact); the copy time is measured and left
    out.  The timed region is the oracle forward."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O

    cpu = host_cpu()
    threads = threads or cpu["affinity_cores"]
    n_sample = min(n_sample, cfg.n_tokens)
    W = O.config_weights(cfg, cache_experts=0)
    x = O.config_x(cfg, rows=np.arange(n_sample))
    routes = O.route(x, W.w_router, W.bias, cfg.top_k)
    need = sorted(set(routes.ids.reshape(-1).tolist()))
    per = cfg.ff_routed * cfg.d_latent
    fr, l, R = cfg.ff_routed, cfg.d_latent, cfg.n_routed
    fetch_s = [0.0]
    if device_experts:
        import torch

        dev = {n: S.gen.device_tensor(cfg, n) for n in ("w_g", "w_u", "w_o")}
        shapes = {"w_g": (R, fr, l), "w_u": (R, fr, l), "w_o": (R, l, fr)}

        def experts(e):
            t0 = time.perf_counter()
            out = tuple(dev[n].reshape(shapes[n])[e].double().cpu().numpy() for n in ("w_g", "w_u", "w_o"))
            fetch_s[0] += time.perf_counter() - t0
            return out
    else:
        stored = {e: tuple(S.to_f64(S.host_tensor(cfg, n, e * per, per), cfg.dtype) for n in ("w_g", "w_u", "w_o"))
                  for e in need}

        def experts(e):  # the oracle reads stored (bf16 / fp32) weights as exact fp64
            g, u, o = stored[e]
            return g.reshape(fr, l), u.reshape(fr, l), o.reshape(l, fr)

    W.experts = experts
    with threadpool_limits(limits=threads, user_api="blas"):
        used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
        t0 = time.perf_counter()
        O.forward(x, W)
        dt = time.perf_counter() - t0 - fetch_s[0]
    src = "device copy of the seeded weights, copy time excluded" if device_experts else "host-generated"
    return {"value": round(n_sample / dt, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"first {n_sample} of {cfg.n_tokens} tokens of {cfg.name} (all five steps, fp64 numpy, "
                      f"{len(need)} routed experts touched ({src}), BLAS threads {used}); {dt:.2f} s",
            "seconds": round(dt, 3), "gflops": round(cfg.flops() * n_sample / cfg.n_tokens / dt / 1e9, 2), **cpu}


def backward_leg(cfg, ids, probs, steps: int, warmup: int):
    """Times latentmoe_routed_backward on the routes of the forward just run,
    with a seeded latent z and upstream gradient du (generated in HBM)."""
    import torch

    import mixture_experts_ffn_sigmoid_amd as M

    N, l, R, f, k = cfg.n_tokens, cfg.d_latent, cfg.n_routed, cfg.ff_routed, cfg.top_k
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = {n: S.gen.device_tensor(cfg, n) for n in ("w_g", "w_u", "w_o", "z", "du")}
    dz = torch.empty((N, l), dtype=torch.float32, device="cuda")
    dprobs = torch.empty((N, k), dtype=torch.float32, device="cuda")
    dw = [torch.empty((R, f, l), dtype=td, device="cuda"), torch.empty((R, f, l), dtype=td, device="cuda"),
          torch.empty((R, l, f), dtype=td, device="cuda")]
    dims = M.dims_of(cfg)
    ws = torch.empty(M.workspace_bytes(dims, M.ENTRY_ROUTED_BACKWARD), dtype=torch.uint8, device="cuda")

    def call():
        M.latentmoe_routed_backward(dims, dev["z"], ids, probs, dev["w_g"], dev["w_u"], dev["w_o"], dev["du"],
                                    dz, dprobs, *dw, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    P = N * k
    es = 2 if cfg.dtype == "bf16" else 4
    flops = 18.0 * P * l * f  # g, up: 4; o: 2; dh: 2; dz: 4; three weight gradients: 6 (x P l f)
    # unavoidable HBM bytes: read the routed weights once, write their gradients once
    wbytes = 3 * R * f * l * es
    by = 2 * wbytes + es * N * l + 4 * N * l * 2
    out = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1), "algorithmic_flops": flops,
           "algorithmic_bytes": by, "hbm_gbs": round(by / ms / 1e6, 1),
           "roofline_frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4),
           "note": "includes recomputing the routed forward quantities and one host sync"}
    del dev, dw, ws
    torch.cuda.empty_cache()
    return out


def layer_backward_leg(cfg, ids, probs, steps: int, warmup: int):
    """Times latentmoe_backward (the whole layer: recomputed forward
    quantities, every weight gradient and dx) on the routes of the forward
    just run, with a seeded upstream gradient dy (generated in HBM)."""
    import torch

    import mixture_experts_ffn_sigmoid_amd as M

    N, d, l, R, f, k = cfg.n_tokens, cfg.d_model, cfg.d_latent, cfg.n_routed, cfg.ff_routed, cfg.top_k
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = S.gen.device_inputs(cfg)
    dy = S.gen.device_tensor(cfg, "dy")
    dx = torch.empty((N, d), dtype=torch.float32, device="cuda")
    grads = {n: torch.empty_like(dev[n]) for n in ("w_down", "w_router", "w_g", "w_u", "w_o", "w_up")}
    if cfg.n_shared:
        grads.update({n: torch.empty_like(dev[n]) for n in ("sh_g", "sh_u", "sh_o")})
    grads["rms_w"] = torch.empty((l,), dtype=torch.float32, device="cuda")
    dims = M.dims_of(cfg)
    ws = torch.empty(M.workspace_bytes(dims, M.ENTRY_BACKWARD), dtype=torch.uint8, device="cuda")

    def call():
        M.latentmoe_backward(dims, dev, dev["x"], ids, probs, dy, dx, grads, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    P = N * k
    nsf = cfg.n_shared * cfg.ff_shared
    # backward products only (the forward's stored quantities are recomputed
    # inside the call and not counted): dr and dh_shared, the routed block
    # (dh 2, dz 4, weight gradients 6, x P l f), dx over [W_down; W_r; S_g; S_u],
    # and the dense weight gradients (w_up, w_down, w_router, shared g/u/o)
    flops = 2.0 * N * d * (l + nsf) + 12.0 * P * l * f + 2.0 * N * d * (l + R + 2 * nsf) \
        + 2.0 * N * d * (2 * l + R + 3 * nsf)
    out = {"ms": round(ms, 4), "tokens_per_s": round(N / ms * 1e3, 1), "tflops": round(flops / ms / 1e9, 1),
           "algorithmic_flops": flops,
           "note": "time includes recomputing z, logits, routed and shared forward quantities, and one host sync; algorithmic flops count the backward products only"}
    del dev, dy, dx, grads, ws
    torch.cuda.empty_cache()
    return out


KERNEL_SOURCES = ("mixture_experts_ffn_sigmoid_amd/csrc/gemm_kernel.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/lmoe_common.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/route_kernels.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/merge_kernels.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/backward_kernels.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/wgrad_kernel.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/lmoe_host.h",
                  "mixture_experts_ffn_sigmoid_amd/csrc/forward.hip",
                  "mixture_experts_ffn_sigmoid_amd/csrc/backward.hip")


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(step: str, workload: str):
    """HBM bytes per launch of `step` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when there is none or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{step}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size (torch's copy kernel), run
    under rocprofv3 --pmc to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def measure_forward(cfg, steps: int, warmup: int) -> dict:
    """Timed forwards on seeded inputs generated in HBM: region 1 (the entry
    point as a user calls it) gives the step time, region 2 (per-step events,
    steps in order on one stream) the per-step times and the roofline of the
    slowest step."""
    import numpy as np
    import torch

    import mixture_experts_ffn_sigmoid_amd as M
    from tests.gpu_util import alloc_forward, device_layer_inputs

    dev = device_layer_inputs(cfg)  # generated in HBM by the seeded generator
    bufs = alloc_forward(cfg)
    W = M.weights_struct(dev)
    torch.cuda.synchronize()

    def fwd_plain():
        M.latentmoe_forward(bufs["dims"], W, dev["x"], bufs["y"], bufs["ids"], bufs["probs"],
                            bufs["counts"], want_capacity=False, workspace=bufs["ws"])

    for _ in range(warmup):
        fwd_plain()
    torch.cuda.synchronize()

    # Timed region 1: K whole-layer forwards as a user calls them (the shared
    # experts overlap the routed experts on a second stream) -> value.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(steps):
        fwd_plain()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / steps

    # Timed region 2: K forwards with per-step events (steps run in order on
    # one stream) -> per-kernel device times and the roofline of the slowest.
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(M.TIMING_EVENTS)]
               for _ in range(steps)]
    for evs in ev_sets:  # torch creates the underlying hipEvent on first record
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    for s in range(steps):
        M.latentmoe_forward_timed(bufs["dims"], W, dev["x"], bufs["y"], bufs["ids"], bufs["probs"],
                                  bufs["counts"], ev_sets[s], workspace=bufs["ws"])
    torch.cuda.synchronize()

    step_ms = {name: float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in ev_sets]))
               for i, name in enumerate(M.STEP_NAMES)}
    counts = bufs["counts"].cpu().numpy()
    C = int(counts.max())
    models = step_models(cfg, counts)
    steps_out = {}
    for name, ms in step_ms.items():
        fl, alg, design = models[name]
        steps_out[name] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                           "gbs": round(alg / ms / 1e6, 1), "design_gbs": round(design / ms / 1e6, 1)}
    dominant = max(step_ms, key=step_ms.get)
    roof = roofline(cfg, dominant, models[dominant], step_ms[dominant])
    layer_bytes = layer_algorithmic_bytes(cfg, counts)
    del dev
    return dict(ms_step=ms_step, step_ms=step_ms, steps_out=steps_out, roof=roof, C=C, t_wall=t_wall,
                bufs=bufs, layer_bytes=layer_bytes, counts=counts)


def roofline(cfg, step: str, model, ms: float) -> dict:
    """Roofline entry of one timed step: MFMA-bound when its FLOPs need more
    time at the MFMA peak than its algorithmic bytes at the HBM peak."""
    fl, alg, design = model
    peak_tf = PEAK_MFMA_TFLOPS[cfg.dtype]
    t = ms / 1e3
    if fl / (peak_tf * 1e12) >= alg / (PEAK_HBM_GBS * 1e9):
        roof = {"kernel": step, "bound": "mfma", "achieved": round(fl / t / 1e12, 1), "peak": peak_tf,
                "unit": "TFLOP/s"}
    else:
        roof = {"kernel": step, "bound": "hbm", "achieved": round(alg / t / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["algorithmic_bytes"] = alg
    roof["design_bytes"] = design
    roof["algorithmic_flops"] = fl
    roof["ms"] = round(ms, 4)
    roof["traffic"] = measured_traffic(step, cfg.name)
    return roof


def secondary_decode(steps: int, warmup: int) -> dict:
    """The few-token weight-streaming layer (full-K3 shapes, 64 tokens): step
    time, tokens/s and the whole layer's algorithmic HBM bytes per step as a
    fraction of the HBM peak, next to the routed gate/up roofline."""
    import torch

    cfg = S.CONFIGS["k3full_n64"]
    fm = measure_forward(cfg, steps, warmup)
    ms = fm["ms_step"]
    out = {"workload": cfg.name, "ms_per_step": round(ms, 4),
           "tokens_per_s": round(cfg.n_tokens / (ms / 1e3), 1),
           "layer_algorithmic_bytes": fm["layer_bytes"],
           "layer_hbm_frac": round(fm["layer_bytes"] / (ms / 1e3) / (PEAK_HBM_GBS * 1e9), 4),
           "roofline": fm["roof"]}
    del fm
    torch.cuda.empty_cache()
    return out


def small_workloads(names, steps: int, warmup: int, cpu: bool) -> dict:
    """The other configured layers (toy fp32, 0.5b, skewed 0.5b): GPU step
    time, tokens/s, TFLOP/s and the fraction of the matching MFMA peak (fp32
    for the toy layer), the roofline of the slowest step, the padded-capacity
    waste R*C / pairs, and the oracle's CPU time on the whole workload (all
    cores; for the toy and 0.5b layers also one thread)."""
    import torch

    out = {}
    for name in names:
        cfg = S.CONFIGS[name]
        fm = measure_forward(cfg, max(steps, 50), warmup)
        ms = fm["ms_step"]
        peak = PEAK_MFMA_TFLOPS[cfg.dtype]
        tf = cfg.flops() / (ms / 1e3) / 1e12
        e = {"ms_per_step": round(ms, 5), "tokens_per_s": round(cfg.n_tokens / (ms / 1e3), 1),
             "tflops": round(tf, 2), "mfma_frac": round(tf / peak, 4), "peak_tflops": peak, "dtype": cfg.dtype,
             "capacity": fm["C"], "padded_over_pairs": round(cfg.n_routed * fm["C"] / cfg.pairs, 3),
             "roofline": fm["roof"], "steps_breakdown": fm["steps_out"]}
        del fm
        torch.cuda.empty_cache()
        if cpu:
            e["cpu_oracle"] = cpu_baseline(cfg, cfg.n_tokens)
            if name in ("toy_n128", "b05_n4096"):
                e["cpu_oracle_1thread"] = cpu_baseline(cfg, cfg.n_tokens, threads=1)
        out[name] = e
    return out


def library_dense(cfg, steps: int, warmup: int) -> dict:
    """The layer's three large dense products as plain library GEMMs
    (torch.mm on ROCm = hipBLASLt), bf16 in and out, fp32 accumulation,
    no epilogue: shared gate/up x [S_g; S_u]^T, the merge [h_sh | u] [S_o |
    W_up]^T and the latent x W_down^T, at the workload's shapes.  A
    comparison for the fused kernels' step times, not part of the layer."""
    import torch

    N, d, l, fs, ns = cfg.n_tokens, cfg.d_model, cfg.d_latent, cfg.ff_shared, cfg.n_shared
    g = torch.Generator(device="cuda").manual_seed(0)
    shapes = {"shared_gateup": (N, d, 2 * ns * fs), "merge_gemm": (N, ns * fs + l, d), "latent_gemm": (N, d, l)}
    out = {}
    for name, (m, k, n) in shapes.items():
        a = torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        b = (torch.randn((n, k), generator=g, device="cuda", dtype=torch.float32) / k ** 0.5).to(torch.bfloat16)
        c = torch.empty((m, n), device="cuda", dtype=torch.bfloat16)
        bt = b.t()  # nn.Linear layout: C = A B^T
        for _ in range(warmup):
            torch.mm(a, bt, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            torch.mm(a, bt, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        fl = 2.0 * m * n * k
        out[name] = {"m": m, "n": n, "k": k, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                     "mfma_frac": round(fl / ms / 1e9 / PEAK_MFMA_TFLOPS["bf16"], 4)}
        del a, b, c, bt
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3full_n8192", choices=sorted(S.CONFIGS))
    ap.add_argument("--cpu-sample", type=int, default=2048, help="tokens for the CPU oracle baseline (0: skip)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward legs (routed block and whole layer)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the few-token (64-token, full-K3) forward measured after the prefill workload")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the toy / 0.5b / skewed 0.5b layers measured after the prefill workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (FETCH_SIZE / WRITE_SIZE calibration)")
    ap.add_argument("--library-dense", action="store_true",
                    help="only time the workload's three large dense products as plain library (hipBLASLt) GEMMs")
    args = ap.parse_args()
    if args.calibrate_copy:
        copy_calibration()
        return
    if args.library_dense:
        print(json.dumps({"workload": args.workload, "library_dense": library_dense(
            S.CONFIGS[args.workload], args.steps, args.warmup)}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer would shard tokens or experts; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_sigmoid_amd as M

    cfg = S.CONFIGS[args.workload]
    M.load()
    fm = measure_forward(cfg, args.steps, args.warmup)
    ms_step, step_ms, steps_out, roof, C, t_wall, bufs = (fm["ms_step"], fm["step_ms"], fm["steps_out"], fm["roof"],
                                                          fm["C"], fm["t_wall"], fm["bufs"])
    peak_tf = PEAK_MFMA_TFLOPS[cfg.dtype]
    flops = cfg.flops()
    tok_s = cfg.n_tokens / (ms_step / 1e3)
    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_sequential": round(sum(step_ms.values()), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_tokens": cfg.n_tokens, "d_model": cfg.d_model,
                   "d_latent": cfg.d_latent, "n_routed": cfg.n_routed, "top_k": cfg.top_k,
                   "n_shared": cfg.n_shared, "ff_routed": cfg.ff_routed, "ff_shared": cfg.ff_shared,
                   "parallelism": "none (1 GPU)"},
        "tflops": round(flops / (ms_step / 1e3) / 1e12, 1),
        "mfma_frac": round(flops / (ms_step / 1e3) / 1e12 / peak_tf, 4),
        "capacity": C,
        "wall_s": round(t_wall, 3),
        "steps_breakdown": steps_out,
        "roofline": roof,
    }
    if not args.no_backward:
        out["routed_backward"] = backward_leg(cfg, bufs["ids"], bufs["probs"], max(2, args.steps // 4), 1)
        out["layer_backward"] = layer_backward_leg(cfg, bufs["ids"], bufs["probs"], max(2, args.steps // 4), 1)
    if args.cpu_sample > 0:
        del bufs, fm
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample, device_experts=cfg.d_latent * cfg.ff_routed > 10**6)
    if cfg.name == "k3full_n8192" and not args.no_secondary:
        fm = bufs = None
        torch.cuda.empty_cache()
        out["secondary"] = secondary_decode(args.steps, args.warmup)
    if cfg.name == "k3full_n8192" and not args.no_small:
        out["workloads"] = small_workloads(("toy_n128", "b05_n4096", "b05skew_n4096"), args.steps, args.warmup,
                                           args.cpu_sample > 0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
