"""CPU oracle of the Stable LatentMoE forward.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
product path (the HIP library and its Python binding) never touches it.  It
shares no code with the GPU path; its only dependency besides numpy is the
seeded input generator ``lmoe_synth`` (used to regenerate large weights
lazily, never for arithmetic).

Everything is plain numpy in fp64.  Stored inputs (fp32, or bf16 bit
patterns) convert to fp64 exactly and no intermediate is rounded.  Library
primitives used as single steps: matrix products, a stable argsort, bincount,
cumsum and ``np.add.at`` (scatter-add).

Citation keys (pages of the K3 repository):
  [sec-07]  raw ``notes/sections/sec-07.tex`` @47c72e5, chapter "SiTU-GLU
            and Stable LatentMoE": the SiTU-GLU equation and property table,
            the component table, the five-step compute flow, the routing code
            and its three notes, the sparse-execution section (permute-
            dispatch + padded bmm) and the load-balancing section.
  [diff]    compare page 584f7e9...main, ``kda/layers/latent_moe.py`` hunks
            (``_routed_u``, ``_route``, ``_balancing_losses``, ``forward``).
  [tests]   same compare page, ``tests/integration/test_k3_arch.py``
            (``_dense_moe_forward`` helper and the MoE tests).

Readings where the pages are silent (each listed in the design notes):
  * RMSNorm is imported but never defined on the pages: here
    ``w * u / sqrt(mean(u^2) + eps)`` with eps inside the square root.
  * Top-k ties: larger ``s+b`` first; equal values go to the lower expert id.
  * The denominator clamp ``max(sum, 1e-9)`` of the routing code is kept.

Pins (tests marked ``not gpu`` in tests/test_oracle_*.py):
  router   closed-form case of the pages' zero-grad test, brute-force sort,
           bias-only-in-selection, all-equal scores (tie rule), k = R.
  dispatch brute-force sort on tiny inputs, counts/offsets/C invariants.
  routed   sparse == dense-then-mask (two independent code paths), identical
           experts, k = R mixture, W_g = 0.
  backward central finite differences of <du, routed_sparse> in every input,
           torch autograd of a dense-then-mask torch composition, exactly
           zero weight gradients for experts without pairs, SiTU derivative
           == torch autograd and its large-beta SwiGLU limit.
  SiTU     |gate * up| < beta1*beta2, near-origin SwiGLU series bound,
           large-beta limit == SwiGLU (torch.nn.functional.silu).
  layer    large-beta layer == a torch library composition (F.linear, F.silu,
           F.rms_norm, torch.topk), token-permutation equivariance,
           linearity in the shared down projection.
  No golden output values are printed on the pages, so absolute outputs of
  the configured layers are pinned only through the above.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import numpy as np

# ---------------------------------------------------------------- SiTU-GLU


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function in fp64, evaluated without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def situ_hidden(a_g: np.ndarray, a_u: np.ndarray, beta1: float, beta2: float) -> np.ndarray:
    """Gated hidden of SiTU-GLU, [sec-07] SiTU-GLU equation:
    gate = beta1*tanh(a_g/beta1)*sigmoid(a_g), up = beta2*tanh(a_u/beta2),
    hidden = gate * up, with a_g = W_g v and a_u = W_u v."""
    gate = beta1 * np.tanh(a_g / beta1) * sigmoid(a_g)
    up = beta2 * np.tanh(a_u / beta2)
    return gate * up


def situ(v: np.ndarray, w_g: np.ndarray, w_u: np.ndarray, w_o: np.ndarray,
         beta1: float, beta2: float) -> np.ndarray:
    """SiTU-GLU expert on rows of v ([M, in] -> [M, in]); weights are
    nn.Linear-shaped [out, in]: w_g, w_u [ff, in], w_o [in, ff]
    ([sec-07] SiTU-GLU equation and listing; no biases)."""
    return situ_hidden(v @ w_g.T, v @ w_u.T, beta1, beta2) @ w_o.T


# ----------------------------------------------------------------- routing


@dataclass
class Routes:
    logits: np.ndarray  # [N, R]  W_r x
    s: np.ndarray       # [N, R]  sigmoid(logits)
    ids: np.ndarray     # [N, k]  int64, descending s+b, ties to the lower id
    p: np.ndarray       # [N, k]  s_i / sum_{j in T} s_j
    margin: np.ndarray  # [N]     (s+b)_(k) - (s+b)_(k+1), +inf when k == R


def route_from_logits(logits: np.ndarray, bias: np.ndarray, k: int) -> Routes:
    """K3 sigmoid routing ("K3 eq.13"), [sec-07] compute-flow step 2 and the
    routing code with its three notes: s = sigmoid(l); T = TopK(s + b, k);
    p_i = s_i / sum_{j in T} s_j.  The bias enters the selection only, p uses
    the raw s; the sum is clamped below at 1e-9 as in the routing code."""
    logits = np.asarray(logits, dtype=np.float64)
    N, R = logits.shape
    if not 1 <= k <= R:
        raise ValueError("need 1 <= k <= R")
    s = sigmoid(logits)
    v = s + np.asarray(bias, dtype=np.float64)[None, :]
    # stable sort of -v: equal values keep ascending expert order
    order = np.argsort(-v, axis=1, kind="stable")
    ids = order[:, :k]
    sel = np.take_along_axis(s, ids, axis=1)
    p = sel / np.maximum(sel.sum(axis=1, keepdims=True), 1e-9)
    if k < R:
        vs = np.take_along_axis(v, order[:, k - 1:k + 1], axis=1)
        margin = vs[:, 0] - vs[:, 1]
    else:
        margin = np.full(N, np.inf)
    return Routes(logits, s, ids.astype(np.int64), p, margin)


def route(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray, k: int) -> Routes:
    """Router on the full-width input: logits = W_r x ([sec-07] component
    table: the router maps d -> n_routed and reads x, not the latent z)."""
    return route_from_logits(x @ w_router.T, bias, k)


def route_softmax_topk(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Legacy router removed by the [diff] forward hunk: ids = top-k of the
    raw logits, weights = softmax over the k selected logits (ties to the
    lower id, as above)."""
    logits = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k]
    sel = np.take_along_axis(logits, ids, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids.astype(np.int64), e / e.sum(axis=1, keepdims=True)


def balancing_losses(logits: np.ndarray, ids: np.ndarray, n_routed: int) -> tuple[float, float]:
    """Unscaled Switch/GShard auxiliary loss and router z-loss, [sec-07]
    load-balancing section: f_e = (#pairs routed to e) / (N k),
    P_e = mean over tokens of sigmoid(l)_e, L_aux = R * sum_e f_e P_e,
    L_z = mean over tokens of (logsumexp_j l_j)^2.  (The layer multiplies
    them by its coefficients, 1e-2 and 1e-3 by default.)"""
    logits = np.asarray(logits, dtype=np.float64)
    counts = np.bincount(np.asarray(ids).reshape(-1), minlength=n_routed).astype(np.float64)
    frac = counts / max(counts.sum(), 1.0)
    prob_mean = sigmoid(logits).mean(axis=0)
    aux = n_routed * float((frac * prob_mean).sum())
    m = logits.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))[:, 0]
    return aux, float(np.mean(lse ** 2))


# ---------------------------------------------------------------- dispatch


@dataclass
class Dispatch:
    counts: np.ndarray     # [R]      pairs per expert
    offsets: np.ndarray    # [R]      exclusive prefix sum of counts
    order: np.ndarray      # [N*k]    flat pair index q = n*k + j, stably sorted by expert
    local_pos: np.ndarray  # [N*k]    position of sorted pair inside its expert
    capacity: int          # C = max counts


def dispatch(ids: np.ndarray, n_routed: int) -> Dispatch:
    """Permute-dispatch bookkeeping, [sec-07] sparse-execution section and
    the [diff] ``_routed_u`` hunk: flatten the (token, slot) pairs in token
    order, stable-sort them by expert id, count pairs per expert, take the
    exclusive prefix sum as offsets, the position inside the expert as
    local_pos and the largest count as the capacity C."""
    eid = np.asarray(ids, dtype=np.int64).reshape(-1)
    order = np.argsort(eid, kind="stable")
    counts = np.bincount(eid, minlength=n_routed)
    offsets = np.cumsum(counts) - counts
    local_pos = np.arange(eid.size) - offsets[eid[order]]
    C = int(counts.max()) if eid.size else 0
    return Dispatch(counts, offsets, order, local_pos, C)


def padded_layout(z: np.ndarray, ids: np.ndarray, n_routed: int, disp: Dispatch | None = None) -> np.ndarray:
    """The [R, C, l] tensor of the sparse-execution section: row local_pos of
    expert e holds z of the token behind that sorted pair; unused rows are 0."""
    if disp is None:
        disp = dispatch(ids, n_routed)
    k = np.asarray(ids).shape[1]
    N, ell = z.shape
    padded = np.zeros((n_routed, disp.capacity, ell), dtype=z.dtype)
    eid = np.asarray(ids, dtype=np.int64).reshape(-1)[disp.order]
    tok = disp.order // k
    padded[eid, disp.local_pos] = z[tok]
    return padded


# ------------------------------------------------------------ routed experts

ExpertFn = Callable[[int], tuple[np.ndarray, np.ndarray, np.ndarray]]


def routed_sparse(z: np.ndarray, ids: np.ndarray, p: np.ndarray, experts: ExpertFn,
                  n_routed: int, beta1: float, beta2: float) -> np.ndarray:
    """u = sum_{i in T} p_i E_i(z), executed the sparse way of the
    sparse-execution section: sort pairs by expert, run each expert on the
    padded block of its pairs, read back only the valid rows, weight them by
    p and scatter-add into token order.  Experts with no pair are skipped
    (their rows would be all padding)."""
    z = np.asarray(z, dtype=np.float64)
    N, ell = z.shape
    k = np.asarray(ids).shape[1]
    u = np.zeros((N, ell), dtype=np.float64)
    if N * k == 0:
        return u
    disp = dispatch(ids, n_routed)
    padded = padded_layout(z, ids, n_routed, disp)
    pw = np.asarray(p, dtype=np.float64).reshape(-1)[disp.order]
    tok = disp.order // k
    eid_sorted = np.asarray(ids, dtype=np.int64).reshape(-1)[disp.order]
    out = np.zeros_like(padded)
    for e in range(n_routed):
        if disp.counts[e] == 0:
            continue
        w_g, w_u, w_o = experts(e)
        out[e] = situ(padded[e], w_g, w_u, w_o, beta1, beta2)
    weighted = pw[:, None] * out[eid_sorted, disp.local_pos]
    np.add.at(u, tok, weighted)
    return u


def routed_dense(z: np.ndarray, ids: np.ndarray, p: np.ndarray, experts: ExpertFn,
                 n_routed: int, beta1: float, beta2: float) -> np.ndarray:
    """Dense reference of the [tests] ``_dense_moe_forward`` helper: run every
    expert on every token, then for each slot j take the selected expert's
    row and add p_j times it.  Cost R*N; tiny inputs only."""
    z = np.asarray(z, dtype=np.float64)
    N, ell = z.shape
    all_out = np.stack([situ(z, *experts(e), beta1, beta2) for e in range(n_routed)], axis=1)
    u = np.zeros((N, ell), dtype=np.float64)
    rows = np.arange(N)
    for j in range(np.asarray(ids).shape[1]):
        u += np.asarray(p)[:, j:j + 1] * all_out[rows, np.asarray(ids)[:, j]]
    return u


# --------------------------------------------------- routed experts, backward


def situ_hidden_grad(a_g: np.ndarray, a_u: np.ndarray, beta1: float,
                     beta2: float) -> tuple[np.ndarray, np.ndarray]:
    """Partial derivatives of the SiTU-GLU hidden h = G(a_g) * U(a_u) of the
    [sec-07] SiTU-GLU equation, G(a) = beta1*tanh(a/beta1)*sigmoid(a) and
    U(a) = beta2*tanh(a/beta2), by the product and chain rules:
        dh/da_g = G'(a_g) U(a_u),  G'(a) = (1 - tanh(a/beta1)^2) sigmoid(a)
                                           + beta1 tanh(a/beta1) sigmoid(a) (1 - sigmoid(a))
        dh/da_u = G(a_g) U'(a_u),  U'(a) = 1 - tanh(a/beta2)^2."""
    a_g = np.asarray(a_g, dtype=np.float64)
    a_u = np.asarray(a_u, dtype=np.float64)
    tg, sg, tu = np.tanh(a_g / beta1), sigmoid(a_g), np.tanh(a_u / beta2)
    gate, up = beta1 * tg * sg, beta2 * tu
    d_gate = (1.0 - tg * tg) * sg + beta1 * tg * sg * (1.0 - sg)
    d_up = 1.0 - tu * tu
    return d_gate * up, gate * d_up


@dataclass
class RoutedGrads:
    dz: np.ndarray      # [N, ell]  dL/dz
    dp: np.ndarray      # [N, k]    dL/dp in slot order
    dw: dict            # e -> (dW_g [ff, ell], dW_u [ff, ell], dW_o [ell, ff])


def routed_backward(z: np.ndarray, ids: np.ndarray, p: np.ndarray, experts: ExpertFn,
                    n_routed: int, beta1: float, beta2: float, du: np.ndarray,
                    want=None, only_want: bool = False) -> RoutedGrads:
    """Reverse-mode derivative of ``routed_sparse`` for an upstream gradient
    du = dL/du [N, ell] (the routed block of the layer backward; the pages
    train this layer and their tests compare its sparse gradients with the
    dense helper's).  For each pair (n, j) with expert e = ids[n, j]:
        forward   a_g = W_g^e z_n, a_u = W_u^e z_n, h = SiTU hidden, o = W_o^e h,
                  u_n += p_nj o
        backward  dp_nj = <du_n, o>,  g_o = p_nj du_n,  dW_o^e += g_o h^T,
                  g_h = (W_o^e)^T g_o,  g_g = g_h * dh/da_g,  g_u = g_h * dh/da_u,
                  dW_g^e += g_g z_n^T,  dW_u^e += g_u z_n^T,
                  dz_n += (W_g^e)^T g_g + (W_u^e)^T g_u.
    Executed per expert over its pairs, the grouping of ``routed_sparse``.
    ``want``: expert ids whose weight gradients are returned (default all);
    an expert with no pair gets exactly zero weight gradients.  With
    ``only_want`` the other experts are skipped altogether (dz and dp then
    hold only the contributions of the wanted experts)."""
    z = np.asarray(z, dtype=np.float64)
    du = np.asarray(du, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    N, ell = z.shape
    k = ids.shape[1]
    pf = np.asarray(p, dtype=np.float64).reshape(-1)
    dz = np.zeros((N, ell), dtype=np.float64)
    dp = np.zeros(N * k, dtype=np.float64)
    want = range(n_routed) if want is None else list(want)
    dw = {}
    disp = dispatch(ids, n_routed) if N * k else None
    for e in range(n_routed):
        if only_want and e not in want:
            continue
        cnt = 0 if disp is None else int(disp.counts[e])
        w_g, w_u, w_o = experts(e) if (cnt or e in want) else (None, None, None)
        if cnt == 0:
            if e in want:
                dw[e] = (np.zeros_like(w_g), np.zeros_like(w_u), np.zeros_like(w_o))
            continue
        q = disp.order[disp.offsets[e]:disp.offsets[e] + cnt]   # flat pair ids of expert e
        tok = q // k
        Z, DU, P = z[tok], du[tok], pf[q]
        a_g, a_u = Z @ w_g.T, Z @ w_u.T
        h = situ_hidden(a_g, a_u, beta1, beta2)
        o = h @ w_o.T
        dp[q] = np.sum(DU * o, axis=1)
        g_o = P[:, None] * DU
        g_h = g_o @ w_o
        dg, dgu = situ_hidden_grad(a_g, a_u, beta1, beta2)
        g_g, g_u = g_h * dg, g_h * dgu
        np.add.at(dz, tok, g_g @ w_g + g_u @ w_u)
        if e in want:
            dw[e] = (g_g.T @ Z, g_u.T @ Z, g_o.T @ h)
    return RoutedGrads(dz, dp.reshape(N, k), dw)


# ------------------------------------------------------------ shared + merge


def shared_sum(x: np.ndarray, sh_g: np.ndarray, sh_u: np.ndarray, sh_o: np.ndarray,
               beta1: float, beta2: float) -> np.ndarray:
    """s_sh = sum_j E_j^sh(x), full-width SiTU experts applied to every
    token and summed in index order ([sec-07] compute-flow step 4)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    for j in range(sh_g.shape[0]):
        out += situ(x, sh_g[j], sh_u[j], sh_o[j], beta1, beta2)
    return out


def rmsnorm(u: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: w * u / sqrt(mean(u^2) + eps).  (The pages
    import RMSNorm without defining it; this is the standard definition.)"""
    u = np.asarray(u, dtype=np.float64)
    return np.asarray(w, dtype=np.float64) * u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)


# ------------------------------------------------------------------- layer


@dataclass
class Weights:
    """fp64 view of the layer's parameters.  ``experts(e)`` returns the routed
    expert's (w_g [f_r,l], w_u [f_r,l], w_o [l,f_r]); it may regenerate them
    lazily so that host memory never holds the full routed set."""
    w_down: np.ndarray    # [l, d]
    w_router: np.ndarray  # [R, d]
    bias: np.ndarray      # [R]
    experts: ExpertFn
    sh_g: np.ndarray      # [n_s, f_s, d]
    sh_u: np.ndarray      # [n_s, f_s, d]
    sh_o: np.ndarray      # [n_s, d, f_s]
    w_up: np.ndarray      # [d, l]
    rms_w: np.ndarray     # [l]
    n_routed: int
    top_k: int
    beta1: float = 4.0
    beta2: float = 25.0
    rms_eps: float = 1e-6


def weights_from_arrays(a: dict, top_k: int, beta1=4.0, beta2=25.0, rms_eps=1e-6) -> Weights:
    """Weights from in-memory fp64 arrays (keys as the input generator names them)."""
    f = lambda n: np.asarray(a[n], dtype=np.float64)  # noqa: E731
    w_g, w_u, w_o = f("w_g"), f("w_u"), f("w_o")
    d = f("w_down").shape[1]
    sh = {n: (f(n) if n in a else np.zeros((0, 1, d))) for n in ("sh_g", "sh_u")}
    sh_o = f("sh_o") if "sh_o" in a else np.zeros((0, d, 1))
    return Weights(f("w_down"), f("w_router"), f("bias"), lambda e: (w_g[e], w_u[e], w_o[e]),
                   sh["sh_g"], sh["sh_u"], sh_o, f("w_up"), f("rms_w"), w_g.shape[0], top_k,
                   beta1, beta2, rms_eps)


def forward(x: np.ndarray, W: Weights, ids: np.ndarray | None = None, dense: bool = False) -> dict:
    """One Stable LatentMoE forward, the five steps of [sec-07] compute flow:
      1. z = W_down x
      2. s = sigmoid(W_r x), T = TopK(s + b, k), p_i = s_i / sum_T s
      3. u = sum_{i in T} p_i E_i^rt(z)          (routed SiTU experts, width l)
      4. s_sh = sum_j E_j^sh(x)                    (shared SiTU experts, width d)
      5. y = s_sh + W_up RMSNorm(u)
    ``ids`` substitutes externally chosen routes (p is then taken from this
    oracle's own s over those ids).  ``dense`` selects the dense-then-mask
    routed path instead of the sparse one."""
    x = np.asarray(x, dtype=np.float64)
    z = x @ W.w_down.T
    r = route(x, W.w_router, W.bias, W.top_k)
    if ids is None:
        ids, p = r.ids, r.p
    else:
        ids = np.asarray(ids, dtype=np.int64)
        sel = np.take_along_axis(r.s, ids, axis=1)
        p = sel / np.maximum(sel.sum(axis=1, keepdims=True), 1e-9)
    fn = routed_dense if dense else routed_sparse
    u = fn(z, ids, p, W.experts, W.n_routed, W.beta1, W.beta2)
    s_sh = shared_sum(x, W.sh_g, W.sh_u, W.sh_o, W.beta1, W.beta2)
    y = s_sh + rmsnorm(u, W.rms_w, W.rms_eps) @ W.w_up.T
    return {"y": y, "z": z, "u": u, "s_sh": s_sh, "ids": ids, "p": p, "routes": r}


def rmsnorm_backward(u: np.ndarray, w: np.ndarray, eps: float, dr: np.ndarray):
    """Reverse-mode derivative of ``rmsnorm`` r = w u rho, rho = (mean(u^2) + eps)^(-1/2):
    du_j = w_j dr_j rho - rho^3 u_j / l * sum_i dr_i w_i u_i,  dw = sum over rows of dr u rho."""
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dr = np.asarray(dr, dtype=np.float64)
    rho = 1.0 / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    dot = np.sum(dr * w * u, axis=-1, keepdims=True)
    du = w * dr * rho - rho ** 3 * u * dot / u.shape[-1]
    return du, np.sum(dr * u * rho, axis=0)


def layer_backward(x: np.ndarray, W: Weights, dy: np.ndarray, ids: np.ndarray | None = None,
                   want=None, only_want: bool = False) -> dict:
    """Reverse-mode derivative of ``forward`` for an upstream gradient dy = dL/dy,
    with the routes held fixed (TopK is piecewise constant; the bias only
    selects and gets no gradient).  Step by step, last forward step first:
      5. y = s_sh + W_up r:       dW_up = dy^T r, dr = dy W_up;  r = RMSNorm(u) -> du, drms_w
      4. s_sh = sum_j S_o^j h_j:  dS_o^j = dy^T h_j, g_h = dy S_o^j, through SiTU to g_g, g_u:
                                  dS_g^j = g_g^T x, dS_u^j = g_u^T x, dx += g_g S_g^j + g_u S_u^j
      3. routed block:            ``routed_backward`` -> dz, dp, dW_g, dW_u, dW_o
      2. p = s_T / sum_T s:       ds_i = (dp_i - sum_T p dp) / sum_T s on T (0 elsewhere),
                                  dl = ds s (1 - s), dW_r = dl^T x, dx += dl W_r
      1. z = W_down x:            dW_down = dz^T x, dx += dz W_down
    ``want`` / ``only_want`` select routed experts as in ``routed_backward``
    (with only_want, dx and the dense gradients miss the other experts' part)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    f = forward(x, W, ids=ids)
    ids, p, u, z = f["ids"], f["p"], f["u"], f["z"]
    s = f["routes"].s
    out = {}
    rn = rmsnorm(u, W.rms_w, W.rms_eps)
    out["w_up"] = dy.T @ rn
    du, out["rms_w"] = rmsnorm_backward(u, W.rms_w, W.rms_eps, dy @ W.w_up)
    dx = np.zeros_like(x)
    gs = {"sh_g": np.zeros_like(W.sh_g), "sh_u": np.zeros_like(W.sh_u), "sh_o": np.zeros_like(W.sh_o)}
    for j in range(W.sh_g.shape[0]):
        a_g, a_u = x @ W.sh_g[j].T, x @ W.sh_u[j].T
        h = situ_hidden(a_g, a_u, W.beta1, W.beta2)
        gs["sh_o"][j] = dy.T @ h
        g_h = dy @ W.sh_o[j]
        dg, dgu = situ_hidden_grad(a_g, a_u, W.beta1, W.beta2)
        g_g, g_u = g_h * dg, g_h * dgu
        gs["sh_g"][j] = g_g.T @ x
        gs["sh_u"][j] = g_u.T @ x
        dx += g_g @ W.sh_g[j] + g_u @ W.sh_u[j]
    out.update(gs)
    rg = routed_backward(z, ids, p, W.experts, W.n_routed, W.beta1, W.beta2, du, want=want,
                         only_want=only_want)
    out["routed"] = rg.dw
    dp = rg.dp
    sel = np.take_along_axis(s, ids, axis=1)
    S = sel.sum(axis=1, keepdims=True)
    Sc = np.maximum(S, 1e-9)
    ds_sel = dp / Sc - (S >= 1e-9) * np.sum(dp * sel, axis=1, keepdims=True) / (Sc * Sc)
    dl = np.zeros_like(s)
    np.put_along_axis(dl, ids, ds_sel * sel * (1.0 - sel), axis=1)
    out["w_router"] = dl.T @ x
    dx += dl @ W.w_router
    out["w_down"] = rg.dz.T @ x
    dx += rg.dz @ W.w_down
    out["x"] = dx
    out["dz"], out["du"], out["dl"] = rg.dz, du, dl
    return out
