"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bars: routing ids equal as sets where the oracle's top-k margin exceeds 1e-4
(valid near-ties otherwise), counts/offsets/order/C and the padded layout
bit-exact on equal routes, y within max|dy|/rms(y_ref) <= 1e-4 (fp32
storage) or 2e-2 (bf16 storage)."""
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


def _small_cfgs():
    base = S.CONFIGS
    return [
        base["toy_n128"],
        base["b05_n4096"],
        base["b05skew_n4096"],
        base["toy_n128"].with_(name="toy_n77_ragged", n_tokens=77),
        base["b05_n4096"].with_(name="b05_n1000_ragged", n_tokens=1000),
        base["toy_n128"].with_(name="toy_noshared", n_shared=0),
        base["toy_n128"].with_(name="toy_n1", n_tokens=1),
        S.LayerConfig("kR_f32", 50, 128, 64, 8, 8, 1, 64, 128, "f32", seed=7),
        S.LayerConfig("kR_bf16", 70, 128, 64, 6, 6, 3, 128, 64, "bf16", seed=8, bias="uniform"),
        S.LayerConfig("wide_k_bf16", 333, 256, 128, 40, 9, 1, 192, 256, "bf16", seed=9, bias="uniform"),
        # few rows with a long K: the latent, router and merge products run split-K
        # (4 slices each, the merge's slices crossing its shared / W_up segment boundary)
        S.LayerConfig("wide_d_bf16_n40", 40, 2048, 256, 16, 4, 1, 256, 2048, "bf16", seed=13, bias="uniform"),
        S.LayerConfig("wide_d_f32_n17", 17, 1024, 128, 16, 2, 1, 128, 1024, "f32", seed=14),
        # the merge product on 256 x 256 tiles with a partly filled last wave:
        # 12 x 32 tiles, 48 per XCD, of which the last 16 run as two K slices
        # of 8 steps (tail split), with ragged rows (2900 = 11 * 256 + 84) and
        # columns (8064 = 31 * 256 + 128)
        S.LayerConfig("tail_split_bf16", 2900, 8064, 128, 8, 2, 1, 128, 896, "bf16", seed=15, bias="uniform"),
    ]


def _forward_parity(cfg, host=None, sample=None):
    """Run the GPU forward and compare y with the oracle on the tokens
    `sample` picks (all by default; a callable gets the GPU ids and the
    near-tie mask).  Full-size layers take their routed weights from the
    device copy of the seeded inputs (checked against the host generator on
    three experts)."""
    _say(f"[forward] {cfg.name} N={cfg.n_tokens}")
    if host is None and cfg.n_tokens * cfg.d_model < 50_000_000 and cfg.n_routed * cfg.ff_routed * cfg.d_latent < 100_000_000:
        host = S.host_inputs(cfg)
    dev = G.device_layer_inputs(cfg, host=host)
    bufs = G.alloc_forward(cfg)
    C = G.run_forward(cfg, dev, bufs)
    ids = bufs["ids"].cpu().numpy()
    counts = bufs["counts"].cpu().numpy()
    probs = bufs["probs"].cpu().numpy().astype(np.float64)
    y = G.download_f64(bufs["y"])

    R = cfg.n_routed
    if host is None:
        G.check_device_copy(cfg, dev, [0, R // 2, R - 1])
        W = G.oracle_weights(cfg, dev)
    else:
        W = O.config_weights(cfg)
    x = O.config_x(cfg)
    routes = O.route(x, W.w_router, W.bias, cfg.top_k)
    near = G.check_routes(ids, routes, W.bias, cfg.top_k)
    assert (counts == np.bincount(ids.reshape(-1), minlength=cfg.n_routed)).all()
    assert C == counts.max()
    if not near.any():
        assert (counts == np.bincount(routes.ids.reshape(-1), minlength=cfg.n_routed)).all()
    # p for the GPU's ids, from the oracle's s
    sel = np.take_along_axis(routes.s, ids, axis=1)
    np.testing.assert_allclose(probs, sel / sel.sum(1, keepdims=True), rtol=0, atol=2e-5)
    if callable(sample):
        sample = sample(ids, near)
    rows = np.arange(cfg.n_tokens) if sample is None else np.asarray(sample)
    t0 = time.perf_counter()
    ref = O.forward(x[rows], W, ids=ids[rows])["y"]
    err = G.rel_err(y[rows], ref)
    _say(f"   C={C} near_ties={int(near.sum())} tokens checked={rows.size} err={err:.3e} "
         f"(oracle {time.perf_counter() - t0:.1f} s)")
    assert err <= G.TOL[cfg.dtype], err
    return dict(y=bufs["y"], C=C, err=err, dev=dev, bufs=bufs, rows=rows)


@pytest.mark.parametrize("cfg", _small_cfgs(), ids=lambda c: c.name)
def test_forward_parity_small(cfg):
    _forward_parity(cfg)


@pytest.mark.parametrize("scale", [1e4, 1e6])
def test_forward_range_guard(scale):
    """bf16 storage keeps z, the p-weighted expert outputs and RMSNorm(u) in
    fp16.  With x scaled up the forward either reports LMOE_ERR_RANGE or
    gives the oracle's y, never a non-finite y with status OK: at x * 1e4, z
    stays below fp16's limit (|z| <= ~5e4) and y must match; at x * 1e6 z
    overflows and both the synchronous forward and the asynchronous one
    followed by latentmoe_forward_check report RANGE."""
    cfg = S.CONFIGS["b05_n4096"]
    _say(f"[range] x * {scale:g}")
    host = dict(S.host_inputs(cfg))
    xs = S.f32_to_bf16_bits(S.bf16_bits_to_f32(host["x"]) * np.float32(scale))
    host["x"] = xs
    dev = G.device_layer_inputs(cfg, host=host)
    bufs = G.alloc_forward(cfg)
    try:
        G.run_forward(cfg, dev, bufs)
        status = 0
    except M.LatentMoEError as e:
        status = e.status
    # the asynchronous form, then the check entry point, agree
    M.latentmoe_forward(bufs["dims"], dev, dev["x"], bufs["y"], bufs["ids"], bufs["probs"], bufs["counts"],
                        want_capacity=False, workspace=bufs["ws"])
    try:
        M.latentmoe_forward_check(bufs["dims"], bufs["ws"])
        status2 = 0
    except M.LatentMoEError as e:
        status2 = e.status
    _say(f"   status {status} / check {status2}")
    assert status2 == status
    if scale >= 1e6:
        assert status == 6
        return
    assert status in (0, 6)
    if status == 6:
        return
    y = G.download_f64(bufs["y"])
    assert np.isfinite(y).all()
    W = O.config_weights(cfg)
    x = S.to_f64(xs, "bf16").reshape(cfg.n_tokens, cfg.d_model)
    routes = O.route(x, W.w_router, W.bias, cfg.top_k)
    ids = bufs["ids"].cpu().numpy()
    near = G.check_routes(ids, routes, W.bias, cfg.top_k)
    ref = O.forward(x, W, ids=ids)["y"]
    err = G.rel_err(y, ref)
    _say(f"   near_ties={int(near.sum())} err={err:.3e}")
    assert err <= G.TOL[cfg.dtype]


def test_forward_is_deterministic():
    cfg = S.CONFIGS["b05skew_n4096"]
    host = S.host_inputs(cfg)
    dev = G.device_layer_inputs(cfg, host=host)
    bufs = G.alloc_forward(cfg)
    G.run_forward(cfg, dev, bufs)
    y1 = bufs["y"].clone()
    G.run_forward(cfg, dev, bufs)
    assert torch.equal(y1.view(torch.int16), bufs["y"].view(torch.int16))


def test_empty_batch_is_noop():
    cfg = S.CONFIGS["toy_n128"].with_(n_tokens=0)
    dims = M.dims_of(cfg)
    dev = G.device_layer_inputs(S.CONFIGS["toy_n128"], host=S.host_inputs(S.CONFIGS["toy_n128"]))
    z = torch.empty(0, device="cuda")
    C = M.latentmoe_forward(dims, dev, z, z, z, z, torch.empty(16, dtype=torch.int32, device="cuda"))
    assert C == 0


@pytest.mark.parametrize("name", ["toy_n128", "b05skew_n4096"])
def test_route_entry(name):
    cfg = S.CONFIGS[name]
    _say(f"[route] {name}")
    host = S.host_inputs(cfg)
    dev = G.device_layer_inputs(cfg, host=host)
    N, R, k = cfg.n_tokens, cfg.n_routed, cfg.top_k
    dims = M.dims_of(cfg)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    probs = torch.empty((N, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((N, R), dtype=torch.float32, device="cuda")
    M.latentmoe_route(dims, dev["x"], dev["w_router"], dev["bias"], ids, probs, logits)
    torch.cuda.synchronize()
    W = O.config_weights(cfg)
    x = O.config_x(cfg)
    routes = O.route(x, W.w_router, W.bias, k)
    l = logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(l - routes.logits)) <= 1e-5 * max(1.0, np.max(np.abs(routes.logits)))
    G.check_routes(ids.cpu().numpy(), routes, W.bias, k)
    # the workspace variant (no logits out) gives the same routes
    ws = torch.empty(M.workspace_bytes(dims, M.ENTRY_ROUTE), dtype=torch.uint8, device="cuda")
    ids2, probs2 = torch.empty_like(ids), torch.empty_like(probs)
    M.latentmoe_route(dims, dev["x"], dev["w_router"], dev["bias"], ids2, probs2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(probs, probs2)


@pytest.mark.parametrize("R,k", [(5, 3), (300, 8), (700, 16), (1500, 8)])
def test_route_expert_counts(R, k):
    """Both routers across expert counts: fewer experts than a wave's lanes,
    several experts per lane, and past 1024.  Sets as in test_route_entry,
    winners in descending order of s + b (softmax: of the logit), weights from
    the chosen scores."""
    cfg = S.LayerConfig(f"route_r{R}", 96, 256, 128, R, k, 1, 64, 256, "bf16", seed=30 + R % 17, bias="uniform")
    _say(f"[route R={R} k={k}]")
    host = S.host_inputs(cfg)
    dev = G.device_layer_inputs(cfg, host=host)
    N = cfg.n_tokens
    dims = M.dims_of(cfg)
    W = O.config_weights(cfg, cache_experts=0)
    x = O.config_x(cfg)
    routes = O.route(x, W.w_router, W.bias, k)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    probs = torch.empty((N, k), dtype=torch.float32, device="cuda")
    M.latentmoe_route(dims, dev["x"], dev["w_router"], dev["bias"], ids, probs, None,
                      torch.empty(M.workspace_bytes(dims, M.ENTRY_ROUTE), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    g = ids.cpu().numpy().astype(np.int64)
    near = G.check_routes(g, routes, W.bias, k)
    v = routes.s + W.bias[None, :]
    gv = np.take_along_axis(v, g, axis=1)
    assert (np.diff(gv[~near], axis=1) <= 1e-6).all()
    gs = np.take_along_axis(routes.s, g, axis=1)
    np.testing.assert_allclose(probs.cpu().numpy(), gs / gs.sum(1, keepdims=True), rtol=0, atol=2e-5)
    # legacy softmax router
    M.latentmoe_route_softmax(dims, dev["x"], dev["w_router"], ids, probs, None,
                              torch.empty(M.workspace_bytes(dims, M.ENTRY_ROUTE), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    lo = x @ W.w_router.T
    o_ids, _ = O.route_softmax_topk(lo, k)
    g = ids.cpu().numpy().astype(np.int64)
    assert ((g >= 0) & (g < R)).all()
    near = _softmax_margin(lo, k) <= G.MARGIN
    assert (np.sort(g[~near], 1) == np.sort(o_ids[~near], 1)).all()
    sel = np.take_along_axis(lo, g, axis=1)
    assert (np.diff(sel[~near], axis=1) <= 1e-6).all()
    e = np.exp(sel - sel.max(1, keepdims=True))
    np.testing.assert_allclose(probs.cpu().numpy(), e / e.sum(1, keepdims=True), rtol=0, atol=2e-5)


def _ids_case(rng, N, R, k, skew=False):
    if skew:  # most tokens pick the same experts
        ids = np.stack([np.arange(k) if rng.random() < 0.8 else rng.permutation(R)[:k] for _ in range(N)])
    else:
        ids = np.stack([rng.permutation(R)[:k] for _ in range(N)])
    return ids.astype(np.int32)


@pytest.mark.parametrize("name", ["k3full_n8192", "toy_n128"])
def test_forward_graph_replay_matches_eager(name):
    """Without the capacity read-back the forward is launches only (no host
    sync, no memset, no allocation), so a caller can capture it in a HIP graph.
    Captured once and replayed three times, with eager work and
    synchronisations between the replays and the outputs poisoned before each:
    every replay equals the eager forward bit for bit (the kernels are
    deterministic).  At the full-K3 prefill size (8192 tokens) the capture
    holds one stream; on the toy layer the shared experts run on the
    library's second stream, forked and joined with events inside the
    capture."""
    cfg = S.CONFIGS[name]
    _say(f"[graph] {cfg.name}")
    dev = G.device_layer_inputs(cfg)
    bufs = G.alloc_forward(cfg)
    W = M.weights_struct(dev)

    def forward():
        M.latentmoe_forward(bufs["dims"], W, dev["x"], bufs["y"], bufs["ids"], bufs["probs"], bufs["counts"],
                            want_capacity=False, workspace=bufs["ws"])

    forward()
    torch.cuda.synchronize()
    names = ("y", "ids", "probs", "counts")
    ref = {n: bufs[n].clone() for n in names}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward()
    torch.cuda.synchronize()
    for rep in range(3):
        bufs["y"].fill_(float("nan"))
        bufs["probs"].fill_(float("nan"))
        bufs["ids"].fill_(-1)
        bufs["counts"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(bufs[n], ref[n]), (rep, n)
        (dev["x"].float() * 2.0).sum().item()  # eager work between replays
    del g


def test_forward_capture_alongside_another_thread():
    """The overlapped path (small shared products) forks onto a second stream
    per host thread: while thread A captures the forward into a graph
    (thread-local capture mode), thread B keeps running eager forwards on its
    own stream.
    B's results and every replay of A's graph equal the eager reference."""
    import threading

    cfg = S.CONFIGS["toy_n128"]
    _say("[graph + thread] toy_n128")
    dev = G.device_layer_inputs(cfg)
    W = M.weights_struct(dev)
    ref_bufs = G.alloc_forward(cfg)
    G.run_forward(cfg, dev, ref_bufs)
    ref = ref_bufs["y"].clone()

    def forward(bufs, stream=None):
        M.latentmoe_forward(bufs["dims"], W, dev["x"], bufs["y"], bufs["ids"], bufs["probs"], bufs["counts"],
                            want_capacity=False, workspace=bufs["ws"], stream=stream)

    b_bufs = G.alloc_forward(cfg)
    b_stream = torch.cuda.Stream()
    started, done = threading.Event(), threading.Event()
    b_ok = []

    def thread_b():
        with torch.cuda.stream(b_stream):
            forward(b_bufs, b_stream)  # creates this thread's side stream before the capture
            b_stream.synchronize()
            started.set()
            for _ in range(20):
                forward(b_bufs, b_stream)
            b_stream.synchronize()
            b_ok.append(torch.equal(b_bufs["y"], ref))
        done.set()

    tb = threading.Thread(target=thread_b)
    tb.start()
    assert started.wait(60)
    a_bufs = G.alloc_forward(cfg)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        forward(a_bufs)
    assert done.wait(60)
    tb.join(60)
    assert b_ok == [True]
    for _ in range(2):
        a_bufs["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a_bufs["y"], ref)
    del g


def test_dispatch_empty_batch():
    """N = 0: C = 0, and counts and offsets come back all zero."""
    R = 16
    dims = M.make_dims(0, 64, 64, R, 2, 0, 64, 0, "bf16")
    counts = torch.full((R,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((R,), 7, dtype=torch.int32, device="cuda")
    none = torch.empty(0, dtype=torch.int32, device="cuda")
    C = M.latentmoe_dispatch(dims, none, None, counts, offsets, none)
    torch.cuda.synchronize()
    assert C == 0
    assert (counts == 0).all() and (offsets == 0).all()


@pytest.mark.parametrize("case", [
    dict(N=128, R=16, k=2, l=128, dt="f32"),
    dict(N=4096, R=16, k=2, l=384, dt="bf16"),
    dict(N=1500, R=37, k=5, l=64, dt="bf16", skew=True),
    dict(N=33, R=4, k=4, l=64, dt="f32"),
    dict(N=1, R=896, k=16, l=128, dt="bf16"),
    dict(N=3000, R=896, k=16, l=64, dt="bf16"),
], ids=lambda c: "N{N}_R{R}_k{k}_{dt}".format(**c))
def test_dispatch_entry_bit_exact(case):
    _say(f"[dispatch] {case}")
    rng = np.random.default_rng(case["N"] + case["R"])
    N, R, k, l, dt = case["N"], case["R"], case["k"], case["l"], case["dt"]
    ids = _ids_case(rng, N, R, k, case.get("skew", False))
    z_host = rng.normal(size=(N, l)).astype(np.float32)
    if dt == "bf16":
        z_host = S.bf16_bits_to_f32(S.f32_to_bf16_bits(z_host))
    dims = M.make_dims(N, 64, l, R, k, 0, 64, 0, dt)
    d_ids = torch.from_numpy(ids).cuda()
    z = torch.from_numpy(z_host).cuda().to(G.torch_dtype(dt))
    counts = torch.empty(R, dtype=torch.int32, device="cuda")
    offsets = torch.empty(R, dtype=torch.int32, device="cuda")
    order = torch.empty(N * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.workspace_bytes(dims, M.ENTRY_DISPATCH), dtype=torch.uint8, device="cuda")
    C = M.latentmoe_dispatch(dims, d_ids, None, counts, offsets, order, workspace=ws)
    ref = O.dispatch(ids, R)
    assert C == ref.capacity
    np.testing.assert_array_equal(counts.cpu().numpy(), ref.counts)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref.offsets)
    np.testing.assert_array_equal(order.cpu().numpy(), ref.order)
    padded = torch.full((R * (C + 3) * l,), float("nan"), dtype=G.torch_dtype(dt), device="cuda")
    C2 = M.latentmoe_dispatch(dims, d_ids, z, counts, offsets, order, padded, C + 3, workspace=ws)
    torch.cuda.synchronize()
    assert C2 == C
    want = O.padded_layout(z_host.astype(np.float64), ids, R, ref)
    got = padded[: R * C * l].float().cpu().numpy().reshape(R, C, l)
    np.testing.assert_array_equal(got, want)
    assert torch.isnan(padded[R * C * l:]).all()  # beyond R*C*l untouched
    if C > 1:
        with pytest.raises(M.LatentMoEError) as ei:
            M.latentmoe_dispatch(dims, d_ids, z, counts, offsets, order, padded, C - 1, workspace=ws)
        assert ei.value.status == 3 and f"C={C}" in str(ei.value)


@pytest.mark.parametrize("name", ["toy_n128", "b05_n4096", "b05skew_n4096"])
def test_experts_entry(name):
    cfg = S.CONFIGS[name]
    _say(f"[experts] {name}")
    rng = np.random.default_rng(3)
    N, R, k, l = cfg.n_tokens, cfg.n_routed, cfg.top_k, cfg.d_latent
    host = S.host_inputs(cfg)
    W = O.config_weights(cfg)
    x = O.config_x(cfg)
    routes = O.route(x, W.w_router, W.bias, k)
    ids = routes.ids.astype(np.int32)
    p = routes.p
    z_host = rng.normal(size=(N, l)).astype(np.float32)
    if cfg.dtype == "bf16":
        z_host = S.bf16_bits_to_f32(S.f32_to_bf16_bits(z_host))
    dims = M.dims_of(cfg)
    dt = G.torch_dtype(cfg.dtype)
    d_ids = torch.from_numpy(ids).cuda()
    z = torch.from_numpy(z_host).cuda().to(dt)
    counts = torch.empty(R, dtype=torch.int32, device="cuda")
    offsets = torch.empty(R, dtype=torch.int32, device="cuda")
    order = torch.empty(N * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(M.workspace_bytes(dims, M.ENTRY_DISPATCH), M.workspace_bytes(dims, M.ENTRY_EXPERTS)),
                     dtype=torch.uint8, device="cuda")
    C = M.latentmoe_dispatch(dims, d_ids, None, counts, offsets, order, workspace=ws)
    padded = torch.empty((R, C, l), dtype=dt, device="cuda")
    M.latentmoe_dispatch(dims, d_ids, z, counts, offsets, order, padded, C, workspace=ws)
    probs = torch.from_numpy(p.astype(np.float32)).cuda()
    u = torch.empty((N, l), dtype=torch.float32, device="cuda")
    dev = G.device_layer_inputs(cfg, host=host)
    M.latentmoe_experts(dims, padded, C, counts, offsets, order, probs, dev["w_g"], dev["w_u"], dev["w_o"],
                        u, workspace=ws)
    torch.cuda.synchronize()
    ref = O.routed_sparse(z_host.astype(np.float64), routes.ids, p.astype(np.float32).astype(np.float64),
                          W.experts, R, cfg.beta1, cfg.beta2)
    err = G.rel_err(u.cpu().numpy().astype(np.float64), ref)
    _say(f"   C={C} err={err:.3e}")
    assert err <= G.TOL_U[cfg.dtype]


@pytest.mark.parametrize("name", ["b05skew_n4096", "toy_n128"])
def test_experts_entry_capacity_below_max_drops_pairs(name):
    """latentmoe_experts with C = max(counts) - 1: the [R, C, l] buffer holds
    each expert's first C pairs, later pairs are dropped, and no read leaves
    the buffer (it sits at the end of a larger allocation whose tail is NaN,
    so a stray read would show up in u).  Reference: the oracle's sparse
    routed sum with the dropped pairs' weights set to 0."""
    cfg = S.CONFIGS[name]
    _say(f"[experts C<max] {name}")
    rng = np.random.default_rng(4)
    N, R, k, l = cfg.n_tokens, cfg.n_routed, cfg.top_k, cfg.d_latent
    host = S.host_inputs(cfg)
    W = O.config_weights(cfg)
    routes = O.route(O.config_x(cfg), W.w_router, W.bias, k)
    ids = routes.ids.astype(np.int32)
    p = routes.p.astype(np.float32)
    z_host = rng.normal(size=(N, l)).astype(np.float32)
    if cfg.dtype == "bf16":
        z_host = S.bf16_bits_to_f32(S.f32_to_bf16_bits(z_host))
    disp = O.dispatch(ids, R)
    Cs = disp.capacity - 1
    assert Cs >= 1
    padded_full = O.padded_layout(z_host.astype(np.float64), ids, R, disp)  # [R, C, l]
    dims = M.dims_of(cfg)
    dt = G.torch_dtype(cfg.dtype)
    buf = torch.full((R * Cs * l + 4096,), float("nan"), dtype=dt, device="cuda")
    padded = buf[4096:].view(R, Cs, l)  # the buffer ends where the allocation ends
    padded.copy_(torch.from_numpy(padded_full[:, :Cs, :].astype(np.float32)).to(dt))
    counts = torch.from_numpy(disp.counts.astype(np.int32)).cuda()
    offsets = torch.from_numpy(disp.offsets.astype(np.int32)).cuda()
    order = torch.from_numpy(disp.order.astype(np.int32)).cuda()
    dev = G.device_layer_inputs(cfg, host=host)
    u = torch.empty((N, l), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.workspace_bytes(dims, M.ENTRY_EXPERTS), dtype=torch.uint8, device="cuda")
    M.latentmoe_experts(dims, padded, Cs, counts, offsets, order, torch.from_numpy(p).cuda(), dev["w_g"],
                        dev["w_u"], dev["w_o"], u, workspace=ws)
    torch.cuda.synchronize()
    kept = np.zeros(N * k, bool)
    kept[disp.order[disp.local_pos < Cs]] = True
    p_kept = np.where(kept.reshape(N, k), p.astype(np.float64), 0.0)
    assert (~kept).sum() >= 1
    ref = O.routed_sparse(z_host.astype(np.float64), routes.ids, p_kept, W.experts, R, cfg.beta1, cfg.beta2)
    got = u.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = G.rel_err(got, ref)
    _say(f"   C={disp.capacity} used C={Cs} dropped={(~kept).sum()} err={err:.3e}")
    assert err <= G.TOL_U[cfg.dtype]


@pytest.mark.slow
def test_experts_entry_k3_prefill_sample():
    """The padded entry points at the full-K3 prefill size: dispatch builds the
    pages' [R, C, l] layout (about 1.2 GB) from a seeded z, and the padded
    grouped GEMMs give u, checked on 1024 stratified tokens (every position of
    every expert's pair list, the most and least loaded experts) against the
    oracle's sparse routed sum (tokens are independent given the routes)."""
    cfg = S.CONFIGS["k3full_n8192"]
    _say(f"[experts full] {cfg.name}")
    N, R, k, l = cfg.n_tokens, cfg.n_routed, cfg.top_k, cfg.d_latent
    dims = M.dims_of(cfg)
    z = S.gen.device_tensor(cfg, "z")
    dev = {n: S.gen.device_tensor(cfg, n) for n in ("w_g", "w_u", "w_o")}
    G.check_device_copy(cfg, dev, [0, R - 1])
    W = G.oracle_weights(cfg, dev)
    routes = O.route(O.config_x(cfg), W.w_router, W.bias, k)
    ids = routes.ids.astype(np.int32)
    p = routes.p.astype(np.float32)
    d_ids = torch.from_numpy(ids).cuda()
    counts = torch.empty(R, dtype=torch.int32, device="cuda")
    offsets = torch.empty(R, dtype=torch.int32, device="cuda")
    order = torch.empty(N * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(M.workspace_bytes(dims, M.ENTRY_DISPATCH), M.workspace_bytes(dims, M.ENTRY_EXPERTS)),
                     dtype=torch.uint8, device="cuda")
    C = M.latentmoe_dispatch(dims, d_ids, None, counts, offsets, order, workspace=ws)
    padded = torch.empty((R, C, l), dtype=G.torch_dtype(cfg.dtype), device="cuda")
    M.latentmoe_dispatch(dims, d_ids, z, counts, offsets, order, padded, C, workspace=ws)
    u = torch.empty((N, l), dtype=torch.float32, device="cuda")
    M.latentmoe_experts(dims, padded, C, counts, offsets, order, torch.from_numpy(p).cuda(), dev["w_g"],
                        dev["w_u"], dev["w_o"], u, workspace=ws)
    torch.cuda.synchronize()
    assert C == int(np.bincount(ids.reshape(-1), minlength=R).max())
    del padded, ws
    rows = G.stratified_tokens(ids, R, 1024)
    z_rows = np.stack([S.to_f64(S.host_tensor(cfg, "z", int(r) * l, l), cfg.dtype) for r in rows])
    t0 = time.perf_counter()
    ref = O.routed_sparse(z_rows, routes.ids[rows], p[rows].astype(np.float64), W.experts, R, cfg.beta1,
                          cfg.beta2)
    err = G.rel_err(G.download_f64(u[torch.as_tensor(rows)]), ref)
    _say(f"   C={C} tokens checked={rows.size} err={err:.3e} (oracle {time.perf_counter() - t0:.1f} s)")
    assert err <= G.TOL_U[cfg.dtype]
    del dev
    torch.cuda.empty_cache()


def test_device_generator_matches_host():
    for name, tensors in [("toy_n128", ["x", "w_g"]), ("b05skew_n4096", ["w_router", "sh_o"]),
                          ("k3full_n64", ["bias", "w_up"])]:
        cfg = S.CONFIGS[name]
        for t in tensors:
            dev = S.gen.device_tensor(cfg, t)
            host = S.host_tensor(cfg, t)
            sdt = S.tensor_spec(cfg, t)[1]
            got = dev.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1) if sdt == "bf16" \
                else dev.cpu().numpy().reshape(-1)
            mism = int((got != host).sum())
            _say(f"[synth] {name}.{t}: {mism} mismatches of {host.size}")
            assert mism == 0


@pytest.mark.slow
def test_forward_parity_k3_decode():
    """The few-token full-K3 layer: y on all 64 tokens."""
    cfg = S.CONFIGS["k3full_n64"]
    r = _forward_parity(cfg, host=None)
    assert r["rows"].size == cfg.n_tokens


@pytest.mark.slow
def test_forward_parity_k3_prefill():
    """The full-K3 prefill layer: y on all 8192 tokens (every row of every
    routed row tile, every near-tie token)."""
    cfg = S.CONFIGS["k3full_n8192"]
    r = _forward_parity(cfg, host=None)
    assert r["rows"].size == cfg.n_tokens
    assert r["C"] >= 131072 // 896


@pytest.mark.slow
def test_forward_parity_k3_past_2g_elements():
    """The largest-size case: the full-K3 layer at N = 70000 tokens, where the
    sorted pair rows of the routed hidden h (N k f_r = 2.29e9 elements) and the
    slot rows (N k l = 4.01e9) run past 2^31.  The sampled tokens are the last
    one (its slot rows are the last) and tokens routed to the two last experts
    (their pairs sit at the end of the sorted order), so the expert GEMMs'
    row offsets, their epilogues and the combine are checked past that point."""
    cfg = S.CONFIGS["k3full_n8192"].with_(name="k3full_n70000", n_tokens=70000)
    N, k, R = cfg.n_tokens, cfg.top_k, cfg.n_routed
    assert N * k * cfg.ff_routed > 2**31 and N * k * cfg.d_latent > 2**31

    def late_pairs(ids, near):
        late = np.flatnonzero((ids >= R - 2).any(axis=1))
        assert late.size >= 2
        strat = G.stratified_tokens(ids, R, 384)  # near-ties are covered at N = 8192
        return np.union1d(strat, [0, int(late[0]), int(late[-1]), N - 1])

    r = _forward_parity(cfg, host=None, sample=late_pairs)
    assert r["C"] >= N * k // R


def _softmax_margin(logits: np.ndarray, k: int) -> np.ndarray:
    R = logits.shape[1]
    if k == R:
        return np.full(logits.shape[0], np.inf)
    part = -np.sort(-logits, axis=1)
    return part[:, k - 1] - part[:, k]


@pytest.mark.parametrize("name", ["toy_n128", "b05skew_n4096", "k3full_n64"])
def test_route_softmax_entry(name):
    """Legacy softmax-top-k router against the oracle's: exact sets where the
    k-th / (k+1)-th logit margin exceeds the near-tie margin, a valid top-k
    otherwise, and softmax weights over the chosen logits."""
    cfg = S.CONFIGS[name]
    _say(f"[route_softmax] {name}")
    dev = G.device_layer_inputs(cfg)
    N, R, k = cfg.n_tokens, cfg.n_routed, cfg.top_k
    dims = M.dims_of(cfg)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    probs = torch.empty((N, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((N, R), dtype=torch.float32, device="cuda")
    M.latentmoe_route_softmax(dims, dev["x"], dev["w_router"], ids, probs, logits)
    torch.cuda.synchronize()
    W = O.config_weights(cfg, cache_experts=0)
    lo = O.config_x(cfg) @ W.w_router.T
    o_ids, _ = O.route_softmax_topk(lo, k)
    g_ids = ids.cpu().numpy().astype(np.int64)
    assert ((g_ids >= 0) & (g_ids < R)).all()
    near = _softmax_margin(lo, k) <= G.MARGIN
    assert (np.sort(g_ids[~near], 1) == np.sort(o_ids[~near], 1)).all()
    for n in np.nonzero(near)[0]:
        vs = np.sort(lo[n])[::-1]
        chosen = np.zeros(R, bool)
        chosen[g_ids[n]] = True
        assert chosen.sum() == k
        assert (lo[n][chosen] >= vs[k - 1] - G.MARGIN).all()
    sel = np.take_along_axis(lo, g_ids, axis=1)
    e = np.exp(sel - sel.max(1, keepdims=True))
    np.testing.assert_allclose(probs.cpu().numpy(), e / e.sum(1, keepdims=True), rtol=0, atol=2e-5)
    # winners come out in descending logit order
    assert (np.diff(sel[~near], axis=1) <= 1e-6).all()
    # the workspace variant gives the same routes
    ws = torch.empty(M.workspace_bytes(dims, M.ENTRY_ROUTE), dtype=torch.uint8, device="cuda")
    ids2, probs2 = torch.empty_like(ids), torch.empty_like(probs)
    M.latentmoe_route_softmax(dims, dev["x"], dev["w_router"], ids2, probs2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(probs, probs2)


@pytest.mark.parametrize("name,n_tokens", [("toy_n128", None), ("toy_n128", 77), ("b05skew_n4096", None),
                                           ("b05_n4096", 1000), ("k3full_n64", None)])
def test_router_losses_entry(name, n_tokens):
    """Auxiliary and z-loss over the forward's own logits and counts, against
    the oracle's (its logits in fp64, the GPU's routes, checked valid)."""
    cfg = S.CONFIGS[name]
    if n_tokens is not None:
        cfg = cfg.with_(name=f"{name}_n{n_tokens}", n_tokens=n_tokens)
    _say(f"[router_losses] {cfg.name}")
    dev = G.device_layer_inputs(cfg)
    N, R, k = cfg.n_tokens, cfg.n_routed, cfg.top_k
    dims = M.dims_of(cfg)
    ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
    probs = torch.empty((N, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((N, R), dtype=torch.float32, device="cuda")
    M.latentmoe_route(dims, dev["x"], dev["w_router"], dev["bias"], ids, probs, logits)
    counts = torch.bincount(ids.reshape(-1).long(), minlength=R).to(torch.int32)
    out = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.router_losses_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    M.latentmoe_router_losses(dims, logits, counts, out, ws)
    torch.cuda.synchronize()
    W = O.config_weights(cfg, cache_experts=0)
    routes = O.route(O.config_x(cfg), W.w_router, W.bias, k)
    g_ids = ids.cpu().numpy()
    G.check_routes(g_ids, routes, W.bias, k)
    aux, zl = O.balancing_losses(routes.logits, g_ids, R)
    got = out.cpu().numpy().astype(np.float64)
    _say(f"   aux {got[0]:.6f} vs {aux:.6f}  z {got[1]:.6f} vs {zl:.6f}")
    assert abs(got[0] - aux) <= 1e-4 * abs(aux)
    assert abs(got[1] - zl) <= 1e-4 * abs(zl) + 1e-6
    # deterministic
    out2 = torch.empty_like(out)
    M.latentmoe_router_losses(dims, logits, counts, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_router_losses_empty_batch():
    cfg = S.CONFIGS["toy_n128"].with_(n_tokens=0)
    dims = M.dims_of(cfg)
    counts = torch.zeros(cfg.n_routed, dtype=torch.int32, device="cuda")
    out = torch.full((2,), 7.0, device="cuda")
    ws = torch.empty(max(M.router_losses_workspace_bytes(dims), 1), dtype=torch.uint8, device="cuda")
    M.latentmoe_router_losses(dims, None, counts, out, ws)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [0.0, 0.0]
