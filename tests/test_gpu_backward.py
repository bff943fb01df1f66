"""Parity of the routed-block backward (latentmoe_routed_backward, through
the C ABI) with the oracle's ``routed_backward`` on seeded inputs: z and du
from the generator, routes from the oracle router on the configured x."""
import time

import numpy as np
import pytest
import torch

import lmoe_synth as S
import mixture_experts_ffn_sigmoid_amd as M
import oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    M.load()  # fails loudly when the library is missing


def _say(*a):
    print(*a, flush=True)


def _routes(cfg, W):
    """ids and fp32 probs from the oracle router on the configured x."""
    r = O.route(O.config_x(cfg), W.w_router, W.bias, cfg.top_k)
    return r.ids.astype(np.int32), r.p.astype(np.float32)


def _run_gpu(cfg, ids, probs, dev=None):
    N, l, R, f, k = cfg.n_tokens, cfg.d_latent, cfg.n_routed, cfg.ff_routed, cfg.top_k
    sdt = cfg.dtype
    if dev is None:  # small configs: host arrays uploaded
        dev = {n: G.upload(S.host_tensor(cfg, n), S.tensor_spec(cfg, n)[1]).reshape(S.tensor_spec(cfg, n)[0])
               for n in ("w_g", "w_u", "w_o", "z", "du")}
    dims = M.dims_of(cfg)
    td = G.torch_dtype(sdt)
    out = dict(
        dz=torch.full((N, l), float("nan"), dtype=torch.float32, device="cuda"),
        dprobs=torch.full((N, k), float("nan"), dtype=torch.float32, device="cuda"),
        dw_g=torch.full((R, f, l), float("nan"), dtype=td, device="cuda"),
        dw_u=torch.full((R, f, l), float("nan"), dtype=td, device="cuda"),
        dw_o=torch.full((R, l, f), float("nan"), dtype=td, device="cuda"),
    )
    ws = torch.empty(max(M.workspace_bytes(dims, M.ENTRY_ROUTED_BACKWARD), 1), dtype=torch.uint8, device="cuda")
    M.latentmoe_routed_backward(dims, dev["z"], torch.from_numpy(ids).cuda(), torch.from_numpy(probs).cuda(),
                                dev["w_g"], dev["w_u"], dev["w_o"], dev["du"], out["dz"], out["dprobs"],
                                out["dw_g"], out["dw_u"], out["dw_o"], workspace=ws)
    torch.cuda.synchronize()
    return out


def _z_du(cfg, rows=None):
    l = cfg.d_latent
    if rows is None:
        z = S.to_f64(S.host_tensor(cfg, "z"), cfg.dtype).reshape(cfg.n_tokens, l)
        du = S.host_tensor(cfg, "du").astype(np.float64).reshape(cfg.n_tokens, l)
        return z, du
    z = np.stack([S.to_f64(S.host_tensor(cfg, "z", int(r) * l, l), cfg.dtype) for r in rows])
    du = np.stack([S.host_tensor(cfg, "du", int(r) * l, l).astype(np.float64) for r in rows])
    return z, du


def _check(name, got, ref, tol):
    err = G.rel_err(got, ref)
    _say(f"   {name}: err {err:.3e}")
    assert np.isfinite(got).all(), name
    assert err <= tol, (name, err)


def _check_wgrad(name, got, ref, dtype):
    """Weight gradients are stored in the storage dtype.  bf16: every element
    within 2 units in the last place of bf16 (2^-7 relative) plus 1e-2 of the
    matrix rms (the fp16 pair intermediates summed over the expert's pairs);
    fp32: the fp32 bar max|diff| <= 1e-4 rms."""
    assert np.isfinite(got).all(), name
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(got - ref)
    if dtype == "bf16":
        bound = 2.0 ** -7 * np.abs(ref) + 1e-2 * rms
        worst = float(np.max(d / bound))
        assert worst <= 1.0, (name, worst, G.rel_err(got, ref))
    else:
        assert G.rel_err(got, ref) <= G.TOL["f32"], (name, G.rel_err(got, ref))
    return G.rel_err(got, ref)


def _cfgs():
    base = S.CONFIGS
    return [
        base["toy_n128"],
        base["b05_n4096"],
        base["b05skew_n4096"],
        base["toy_n128"].with_(name="toy_n77_ragged", n_tokens=77),
        base["toy_n128"].with_(name="toy_n3_sparse", n_tokens=3),
        S.LayerConfig("kR_bf16", 70, 128, 64, 6, 6, 3, 128, 64, "bf16", seed=8, bias="uniform"),
        S.LayerConfig("wide_k_bf16", 333, 256, 128, 40, 9, 1, 192, 256, "bf16", seed=9, bias="uniform"),
        # 256-multiple widths with every padded pair count 0/64/128/192 (largest 182):
        # the strip weight-gradient kernel; 420 tokens push one expert to 194
        # pairs and the batched GEMM path instead; l = 512 gives dW_o two
        # 256-row strips and dW_g, dW_u four column tiles (same routes)
        _STRIP,
        _STRIP.with_(name="strip_over_bf16", n_tokens=420),
        _STRIP.with_(name="strip_wide_bf16", d_latent=512),
    ]


_STRIP = S.LayerConfig("strip_bf16", 400, 256, 256, 24, 2, 1, 256, 256, "bf16", seed=11, bias="quadratic",
                       router_skew_rows=3, router_skew=2.5)


@pytest.mark.parametrize("cfg", _cfgs(), ids=lambda c: c.name)
def test_routed_backward_parity(cfg):
    _say(f"[routed_backward] {cfg.name}")
    W = O.config_weights(cfg, cache_experts=cfg.n_routed)
    ids, probs = _routes(cfg, W)
    out = _run_gpu(cfg, ids, probs)
    z, du = _z_du(cfg)
    ref = O.routed_backward(z, ids, probs.astype(np.float64), W.experts, cfg.n_routed, cfg.beta1, cfg.beta2, du)
    tol = G.TOL[cfg.dtype]
    _check("dz", G.download_f64(out["dz"]), ref.dz, tol)
    _check("dprobs", G.download_f64(out["dprobs"]), ref.dp, tol)
    used = set(ids.reshape(-1).tolist())
    for e in range(cfg.n_routed):
        for j, nm in enumerate(("dw_g", "dw_u", "dw_o")):
            got = G.download_f64(out[nm][e])
            if e not in used:  # experts without pairs: exact zeros
                assert np.all(got == 0.0), (nm, e)
            else:
                _check_wgrad(f"{nm}[{e}]", got, ref.dw[e][j], cfg.dtype)
    _say(f"   experts used {len(used)}/{cfg.n_routed}")


def test_routed_backward_is_deterministic():
    cfg = S.CONFIGS["b05skew_n4096"]
    W = O.config_weights(cfg)
    ids, probs = _routes(cfg, W)
    a = _run_gpu(cfg, ids, probs)
    b = _run_gpu(cfg, ids, probs)
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]), k


def test_routed_backward_empty_batch_zeroes_weight_grads():
    cfg = S.CONFIGS["toy_n128"].with_(name="toy_n0", n_tokens=0)
    out = _run_gpu(cfg, np.zeros((0, cfg.top_k), np.int32), np.zeros((0, cfg.top_k), np.float32),
                   dev={n: G.upload(S.host_tensor(S.CONFIGS["toy_n128"], n), "f32").reshape(
                       S.tensor_spec(S.CONFIGS["toy_n128"], n)[0]) for n in ("w_g", "w_u", "w_o")} |
                   {"z": torch.empty(0, device="cuda"), "du": torch.empty(0, device="cuda")})
    for nm in ("dw_g", "dw_u", "dw_o"):
        assert torch.all(out[nm] == 0)


def _full_size(name, tok_sample, n_experts_sample):
    """The routed block at a full-K3 size: dz and dprobs on the tokens
    `tok_sample` picks (a list, or a callable of the routes), the weight
    gradients of sampled experts over all their pairs, exact zeros for an
    expert without pairs.  The oracle reads the routed weights from the
    device copy (checked against the host generator on three experts)."""
    cfg = S.CONFIGS[name] if isinstance(name, str) else name
    _say(f"[routed_backward full] {cfg.name}")
    R = cfg.n_routed
    dev = {n: S.gen.device_tensor(cfg, n) for n in ("w_g", "w_u", "w_o", "z", "du")}
    G.check_device_copy(cfg, dev, [0, R // 2, R - 1])
    W = G.oracle_weights(cfg, dev)
    ids, probs = _routes(cfg, W)
    out = _run_gpu(cfg, ids, probs, dev=dev)
    del dev["z"], dev["du"]
    tol = G.TOL[cfg.dtype]
    # dz / dprobs of sampled tokens: their own pairs only
    rows = np.asarray(tok_sample(ids) if callable(tok_sample) else tok_sample)
    z, du = _z_du(cfg, rows)
    t0 = time.perf_counter()
    ref = O.routed_backward(z, ids[rows], probs[rows].astype(np.float64), W.experts, cfg.n_routed,
                            cfg.beta1, cfg.beta2, du, want=[])
    _say(f"   {rows.size} tokens (oracle {time.perf_counter() - t0:.1f} s)")
    _check("dz (sampled tokens)", G.download_f64(out["dz"][torch.as_tensor(rows)]), ref.dz, tol)
    _check("dprobs (sampled tokens)", G.download_f64(out["dprobs"][torch.as_tensor(rows)]), ref.dp, tol)
    # weight gradients of sampled experts: all their pairs
    counts = np.bincount(ids.reshape(-1), minlength=cfg.n_routed)
    used = np.nonzero(counts)[0]
    picks = [int(used[0]), int(used[len(used) // 2]), int(used[-1])][:n_experts_sample]
    for e in picks:
        toks = np.nonzero((ids == e).any(axis=1))[0]
        z, du = _z_du(cfg, toks)
        r = O.routed_backward(z, ids[toks], probs[toks].astype(np.float64), W.experts, cfg.n_routed,
                              cfg.beta1, cfg.beta2, du, want=[e], only_want=True)
        for j, nm in enumerate(("dw_g", "dw_u", "dw_o")):
            err = _check_wgrad(f"{nm}[{e}]", G.download_f64(out[nm][e]), r.dw[e][j], cfg.dtype)
            _say(f"   {nm}[{e}] ({counts[e]} pairs): err {err:.3e}")
    empty = np.nonzero(counts == 0)[0]
    if empty.size:
        for nm in ("dw_g", "dw_u", "dw_o"):
            assert torch.all(out[nm][int(empty[0])].float() == 0), nm
    del dev, out
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_routed_backward_k3_decode_sample():
    """Few-token full-K3 shape: dz and dprobs on all 64 tokens."""
    _full_size("k3full_n64", list(range(64)), 3)


@pytest.mark.slow
def test_routed_backward_k3_prefill_sample():
    """Prefill full-K3 shape: dz and dprobs on 1024 stratified tokens."""
    _full_size("k3full_n8192", lambda ids: G.stratified_tokens(ids, 896, 1024), 2)


@pytest.mark.slow
def test_routed_backward_k3_past_2g_elements():
    """The largest size: the full-K3 routed block at N = 70000 tokens, where the
    per-pair buffers (h and the gate / up pre-activations, N k f_r = 2.29e9
    elements; the expert outputs, N k l = 4.01e9) pass 2^31.  Sampled: the last
    token, tokens routed to the two last experts (their pairs sit at the end
    of the sorted order) and 256 stratified tokens, and the weight gradients
    of the first, a middle and the last expert over all their pairs."""
    cfg = S.CONFIGS["k3full_n8192"].with_(name="k3full_n70000", n_tokens=70000)
    N, R = cfg.n_tokens, cfg.n_routed

    def late_pairs(ids):
        late = np.flatnonzero((ids >= R - 2).any(axis=1))
        return np.union1d(G.stratified_tokens(ids, R, 256), [int(late[0]), int(late[-1]), N - 1])

    _full_size(cfg, late_pairs, 3)
    torch.cuda.empty_cache()


# ------------------------------------------------------------ whole layer


def _layer_cfgs():
    base = S.CONFIGS
    return [
        base["toy_n128"],
        base["b05_n4096"],
        base["b05skew_n4096"],
        base["toy_n128"].with_(name="toy_n77_ragged", n_tokens=77),
        base["toy_n128"].with_(name="toy_noshared", n_shared=0),
        S.LayerConfig("kR_bf16", 70, 128, 64, 6, 6, 3, 128, 64, "bf16", seed=8, bias="uniform"),
        S.LayerConfig("wide_k_bf16", 333, 256, 128, 40, 9, 1, 192, 256, "bf16", seed=9, bias="uniform"),
        _STRIP,
        # dx on 256 x 256 tiles (12 x 32, 48 per XCD) whose last 16 tiles per
        # XCD run as two K slices (tail split), ragged in rows and columns
        S.LayerConfig("tail_split_bf16", 2900, 8064, 128, 8, 2, 1, 128, 896, "bf16", seed=15, bias="uniform"),
    ]


def _grad_bufs(cfg):
    N, d, l, R, f = cfg.n_tokens, cfg.d_model, cfg.d_latent, cfg.n_routed, cfg.ff_routed
    td = G.torch_dtype(cfg.dtype)
    nan = float("nan")
    g = {n: torch.full(S.tensor_spec(cfg, n)[0], nan, dtype=td, device="cuda")
         for n in ("w_down", "w_router", "w_g", "w_u", "w_o", "w_up")}
    if cfg.n_shared > 0:
        for n in ("sh_g", "sh_u", "sh_o"):
            g[n] = torch.full(S.tensor_spec(cfg, n)[0], nan, dtype=td, device="cuda")
    g["rms_w"] = torch.full((l,), nan, dtype=torch.float32, device="cuda")
    return g


def _run_layer_gpu(cfg, ids, probs, dev):
    N, d = cfg.n_tokens, cfg.d_model
    dims = M.dims_of(cfg)
    dx = torch.full((N, d), float("nan"), dtype=torch.float32, device="cuda")
    grads = _grad_bufs(cfg)
    ws = torch.empty(max(M.workspace_bytes(dims, M.ENTRY_BACKWARD), 1), dtype=torch.uint8, device="cuda")
    M.latentmoe_backward(dims, dev, dev["x"], torch.from_numpy(ids).cuda(), torch.from_numpy(probs).cuda(),
                         dev["dy"], dx, grads, workspace=ws)
    torch.cuda.synchronize()
    return dx, grads


def _layer_routes(cfg, W, x=None):
    x = O.config_x(cfg) if x is None else x
    r = O.route(x, W.w_router, W.bias, cfg.top_k)
    return r.ids.astype(np.int32), r.p.astype(np.float32)


@pytest.mark.parametrize("cfg", _layer_cfgs(), ids=lambda c: c.name)
def test_layer_backward_parity(cfg):
    _say(f"[layer_backward] {cfg.name}")
    host = S.host_inputs(cfg)
    dev = G.device_layer_inputs(cfg, host=host)
    dev["dy"] = G.upload(S.host_tensor(cfg, "dy"), cfg.dtype).reshape(cfg.n_tokens, cfg.d_model)
    W = O.config_weights(cfg, cache_experts=cfg.n_routed)
    x = O.config_x(cfg)
    ids, probs = _layer_routes(cfg, W, x)
    dx, grads = _run_layer_gpu(cfg, ids, probs, dev)
    dy = S.to_f64(S.host_tensor(cfg, "dy"), cfg.dtype).reshape(cfg.n_tokens, cfg.d_model)
    ref = O.layer_backward(x, W, dy, ids=ids)
    _check("dx", G.download_f64(dx), ref["x"], G.TOL[cfg.dtype])
    names = ["w_down", "w_router", "w_up"] + (["sh_g", "sh_u", "sh_o"] if cfg.n_shared else [])
    for n in names:
        err = _check_wgrad(n, G.download_f64(grads[n]).reshape(ref[n].shape), ref[n], cfg.dtype)
        _say(f"   {n}: err {err:.3e}")
    _check("rms_w", G.download_f64(grads["rms_w"]), ref["rms_w"], G.TOL[cfg.dtype])
    used = set(ids.reshape(-1).tolist())
    for e in range(cfg.n_routed):
        for j, n in enumerate(("w_g", "w_u", "w_o")):
            got = G.download_f64(grads[n][e])
            if e not in used:
                assert np.all(got == 0.0), (n, e)
            else:
                _check_wgrad(f"{n}[{e}]", got, ref["routed"][e][j], cfg.dtype)


def test_layer_backward_empty_batch():
    cfg = S.CONFIGS["toy_n128"].with_(name="toy_n0", n_tokens=0)
    base = S.CONFIGS["toy_n128"]
    dev = G.device_layer_inputs(base, host=S.host_inputs(base))
    dims = M.dims_of(cfg)
    grads = _grad_bufs(cfg)
    ws = torch.empty(max(M.workspace_bytes(dims, M.ENTRY_BACKWARD), 1), dtype=torch.uint8, device="cuda")
    e = torch.empty(0, device="cuda")
    M.latentmoe_backward(dims, dev, e, e, e, e, e, grads, workspace=ws)
    torch.cuda.synchronize()
    for n, t in grads.items():
        assert torch.all(t == 0), n


@pytest.mark.slow
def test_layer_backward_k3_decode_full():
    """Full-K3 decode shape: dx and every gradient except the routed experts'
    (sampled experts, all their pairs)."""
    cfg = S.CONFIGS["k3full_n64"]
    _say(f"[layer_backward full] {cfg.name}")
    dev = G.device_layer_inputs(cfg)
    dev["dy"] = S.gen.device_tensor(cfg, "dy")
    G.check_device_copy(cfg, dev, [0, cfg.n_routed - 1])
    W = G.oracle_weights(cfg, dev)
    x = O.config_x(cfg)
    ids, probs = _layer_routes(cfg, W)
    dx, grads = _run_layer_gpu(cfg, ids, probs, dev)
    dy = S.to_f64(S.host_tensor(cfg, "dy"), cfg.dtype).reshape(cfg.n_tokens, cfg.d_model)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.n_routed)
    used = np.nonzero(counts)[0]
    picks = [int(used[0]), int(used[len(used) // 2])]
    ref = O.layer_backward(x, W, dy, ids=ids, want=picks)
    _check("dx", G.download_f64(dx), ref["x"], G.TOL[cfg.dtype])
    for n in ("w_down", "w_router", "w_up", "sh_g", "sh_u", "sh_o"):
        err = _check_wgrad(n, G.download_f64(grads[n]).reshape(ref[n].shape), ref[n], cfg.dtype)
        _say(f"   {n}: err {err:.3e}")
    _check("rms_w", G.download_f64(grads["rms_w"]), ref["rms_w"], G.TOL[cfg.dtype])
    for e in picks:
        for j, n in enumerate(("w_g", "w_u", "w_o")):
            _check_wgrad(f"{n}[{e}]", G.download_f64(grads[n][e]), ref["routed"][e][j], cfg.dtype)


@pytest.mark.slow
def test_layer_backward_k3_prefill_sample():
    """Full-K3 prefill shape: dx of 1024 stratified tokens (tokens are
    independent given the routes, so the oracle runs on those rows alone)."""
    cfg = S.CONFIGS["k3full_n8192"]
    _say(f"[layer_backward full] {cfg.name}")
    dev = G.device_layer_inputs(cfg)
    dev["dy"] = S.gen.device_tensor(cfg, "dy")
    G.check_device_copy(cfg, dev, [0, cfg.n_routed - 1])
    W = G.oracle_weights(cfg, dev)
    ids, probs = _layer_routes(cfg, W, O.config_x(cfg))
    dx, grads = _run_layer_gpu(cfg, ids, probs, dev)
    del grads
    rows = G.stratified_tokens(ids, cfg.n_routed, 1024)
    x = O.config_x(cfg, rows=rows)
    d = cfg.d_model
    dy = np.stack([S.to_f64(S.host_tensor(cfg, "dy", int(r) * d, d), cfg.dtype) for r in rows])
    t0 = time.perf_counter()
    ref = O.layer_backward(x, W, dy, ids=ids[rows], want=[])
    _say(f"   {rows.size} tokens (oracle {time.perf_counter() - t0:.1f} s)")
    _check("dx (sampled tokens)", G.download_f64(dx[torch.as_tensor(rows)]), ref["x"], G.TOL[cfg.dtype])
    del dev
    torch.cuda.empty_cache()


def test_layer_backward_is_deterministic():
    cfg = S.CONFIGS["b05skew_n4096"]
    host = S.host_inputs(cfg)
    dev = G.device_layer_inputs(cfg, host=host)
    dev["dy"] = G.upload(S.host_tensor(cfg, "dy"), cfg.dtype).reshape(cfg.n_tokens, cfg.d_model)
    W = O.config_weights(cfg)
    ids, probs = _layer_routes(cfg, W)
    a = _run_layer_gpu(cfg, ids, probs, dev)
    b = _run_layer_gpu(cfg, ids, probs, dev)
    assert torch.equal(a[0], b[0])
    for n in a[1]:
        t, u = a[1][n], b[1][n]
        if t.dtype == torch.bfloat16:
            t, u = t.view(torch.int16), u.view(torch.int16)
        assert torch.equal(t, u), n
