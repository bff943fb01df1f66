"""fp64 weights of a configured layer for the oracle (test infrastructure).

Small configurations are materialised whole.  For the full-K3 shapes the
routed experts (tens of GB) are regenerated one expert at a time from the
seeded generator when the oracle asks for them, so host memory holds only
the dense weights and a few experts.
"""
from __future__ import annotations

from collections import OrderedDict

import numpy as np

import lmoe_synth as S

from .latentmoe_oracle import Weights


def _f64(cfg, name, start=0, count=None):
    sdt = S.tensor_spec(cfg, name)[1]
    return S.to_f64(S.host_tensor(cfg, name, start, count), sdt)


def config_x(cfg, rows=None) -> np.ndarray:
    """Input tokens [N, d] (or only the given token rows) in fp64."""
    d = cfg.d_model
    if rows is None:
        return _f64(cfg, "x").reshape(cfg.n_tokens, d)
    rows = np.asarray(rows, dtype=np.int64)
    return np.stack([_f64(cfg, "x", int(r) * d, d) for r in rows]) if rows.size else np.zeros((0, d))


def config_weights(cfg, cache_experts: int = 4) -> Weights:
    R, l, fr = cfg.n_routed, cfg.d_latent, cfg.ff_routed
    shape = lambda n: S.tensor_spec(cfg, n)[0]  # noqa: E731
    dense = {n: _f64(cfg, n).reshape(shape(n)) for n in ("w_down", "w_router", "w_up")}
    bias = S.host_tensor(cfg, "bias").astype(np.float64)
    rms_w = S.host_tensor(cfg, "rms_w").astype(np.float64)
    if cfg.n_shared > 0:
        sh = {n: _f64(cfg, n).reshape(shape(n)) for n in ("sh_g", "sh_u", "sh_o")}
    else:
        d = cfg.d_model
        sh = {"sh_g": np.zeros((0, 1, d)), "sh_u": np.zeros((0, 1, d)), "sh_o": np.zeros((0, d, 1))}
    per = fr * l
    cache: OrderedDict = OrderedDict()

    def experts(e: int):
        if e in cache:
            cache.move_to_end(e)
            return cache[e]
        w = (_f64(cfg, "w_g", e * per, per).reshape(fr, l),
             _f64(cfg, "w_u", e * per, per).reshape(fr, l),
             _f64(cfg, "w_o", e * per, per).reshape(l, fr))
        cache[e] = w
        if len(cache) > cache_experts:
            cache.popitem(last=False)
        return w

    return Weights(dense["w_down"], dense["w_router"], bias, experts, sh["sh_g"], sh["sh_u"],
                   sh["sh_o"], dense["w_up"], rms_w, R, cfg.top_k, cfg.beta1, cfg.beta2, cfg.rms_eps)
