"""Layer configurations and the input recipe.

Shapes follow the Stable LatentMoE layer of the K3 notes (raw
``notes/sections/sec-07.tex`` @47c72e5, component table and shape overview):
x [N,d]; W_down [l,d]; W_r [R,d]; expert bias b [R]; routed SiTU experts
W_g, W_u [R,f_r,l] and W_o [R,l,f_r] (stacked ``nn.Linear`` weights, [out,in]);
shared SiTU experts [n_s,f_s,d] / [n_s,d,f_s]; RMSNorm weight [l]; W_up [d,l].
The toy / 0.5b / full-K3 widths come from the K3 size table (``sec-08.tex``
@5a7d949, subsection on toy sizes) and from the 0.5b preset of the config
diff (``k3_config.py``); the expert inner widths and token counts are the
workload definitions of this project.

Every weight is drawn N(0, 1/fan_in), x ~ N(0, 1) (the layer sees the output
of a pre-norm, so unit RMS is its natural input scale), RMSNorm weight = 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    n_tokens: int
    d_model: int
    d_latent: int
    n_routed: int
    top_k: int
    n_shared: int
    ff_routed: int
    ff_shared: int
    dtype: str  # "f32" or "bf16": storage type of x, weights and y
    seed: int
    bias: str = "zero"  # "zero" | "quadratic" (0.5*(i/(R-1))^2) | "uniform" (U(-0.01, 0.01))
    router_skew_rows: int = 0  # router rows 0..rows-1 are multiplied by router_skew
    router_skew: float = 1.0
    beta1: float = 4.0
    beta2: float = 25.0
    rms_eps: float = 1e-6
    description: str = field(default="", compare=False)

    def with_tokens(self, n_tokens: int) -> "LayerConfig":
        return replace(self, n_tokens=n_tokens)

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.n_tokens * self.top_k

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward (2 per multiply-add, routed work over
        the N*k token-expert pairs, padding not counted)."""
        N, d, l, R, k = self.n_tokens, self.d_model, self.d_latent, self.n_routed, self.top_k
        dense = N * (2 * d * l + 2 * d * R + 2 * l * d + 6 * self.n_shared * d * self.ff_shared)
        routed = 6 * N * k * l * self.ff_routed
        return float(dense + routed)


CONFIGS: dict[str, LayerConfig] = {
    c.name: c
    for c in [
        LayerConfig(
            "toy_n128", 128, 256, 128, 16, 2, 1, 256, 512, "f32", seed=0,
            description="toy LatentMoE layer, fp32, N=128 (B=2, T=64)",
        ),
        LayerConfig(
            "b05_n4096", 4096, 768, 384, 16, 2, 2, 768, 2048, "bf16", seed=1,
            description="0.5b-preset layer, bf16 storage, fp32 accumulate, N=4096 (B=2, T=2048)",
        ),
        LayerConfig(
            "b05skew_n4096", 4096, 768, 384, 16, 2, 2, 768, 2048, "bf16", seed=2,
            bias="quadratic", router_skew_rows=4, router_skew=3.0,
            description="0.5b layer with skewed routing: b_i=0.5(i/15)^2, router rows 0-3 x3, N=4096",
        ),
        LayerConfig(
            "k3full_n64", 64, 7168, 3584, 896, 16, 1, 2048, 18432, "bf16", seed=3, bias="uniform",
            description="full-K3-shaped layer, few-token weight-streaming regime, N=64",
        ),
        LayerConfig(
            "k3full_n8192", 8192, 7168, 3584, 896, 16, 1, 2048, 18432, "bf16", seed=4,
            description="full-K3-shaped layer, prefill regime, N=8192 (B=4, T=2048)",
        ),
    ]
}

# Stream ids of the generator, one per tensor.
TENSOR_IDS = {
    "x": 1, "w_down": 2, "w_router": 3, "w_g": 4, "w_u": 5, "w_o": 6,
    "sh_g": 7, "sh_u": 8, "sh_o": 9, "w_up": 10, "bias": 11,
    # inputs of the backward: a latent z and upstream gradients du (routed block), dy (layer)
    "z": 12, "du": 13, "dy": 14,
}


def tensor_names(cfg: LayerConfig) -> list[str]:
    names = ["x", "w_down", "w_router", "bias", "w_g", "w_u", "w_o"]
    if cfg.n_shared > 0:
        names += ["sh_g", "sh_u", "sh_o"]
    return names + ["w_up", "rms_w"]


def tensor_spec(cfg: LayerConfig, name: str):
    """(shape, storage dtype, scale, row_len, rows_mult, row_mult) of one input."""
    N, d, l, R = cfg.n_tokens, cfg.d_model, cfg.d_latent, cfg.n_routed
    fr, fs, ns = cfg.ff_routed, cfg.ff_shared, cfg.n_shared
    dt = cfg.dtype
    s = lambda fan_in: 1.0 / math.sqrt(fan_in)  # noqa: E731
    table = {
        "x": ((N, d), dt, 1.0),
        "w_down": ((l, d), dt, s(d)),
        "w_router": ((R, d), dt, s(d)),
        "w_g": ((R, fr, l), dt, s(l)),
        "w_u": ((R, fr, l), dt, s(l)),
        "w_o": ((R, l, fr), dt, s(fr)),
        "sh_g": ((ns, fs, d), dt, s(d)),
        "sh_u": ((ns, fs, d), dt, s(d)),
        "sh_o": ((ns, d, fs), dt, s(fs)),
        "w_up": ((d, l), dt, s(l)),
        "bias": ((R,), "f32", None),
        "rms_w": ((l,), "f32", None),
        "z": ((N, l), dt, 1.0),
        "du": ((N, l), "f32", 1.0),
        "dy": ((N, d), dt, 1.0),
    }
    shape, sdt, scale = table[name]
    if name == "w_router" and cfg.router_skew_rows > 0:
        return shape, sdt, scale, d, cfg.router_skew_rows, cfg.router_skew
    return shape, sdt, scale, 0, 0, 1.0
