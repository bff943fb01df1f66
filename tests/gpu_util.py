"""Helpers of the GPU parity tests: upload seeded inputs, run the C ABI,
compare with the oracle under the near-tie routing rule."""
from __future__ import annotations

import numpy as np
import torch

import lmoe_synth as S
import mixture_experts_ffn_sigmoid_amd as M

MARGIN = 1e-4  # routing sets must match exactly where the top-k margin exceeds this


def torch_dtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def upload(arr: np.ndarray, dt: str, device="cuda") -> torch.Tensor:
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def download_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_layer_inputs(cfg, device="cuda", host: dict | None = None) -> dict:
    """All inputs of cfg in device memory.  Small configs go through the host
    arrays (also handed to the oracle); large ones are generated on the GPU."""
    out = {}
    for name in S.tensor_names(cfg):
        sdt = S.tensor_spec(cfg, name)[1]
        if host is not None:
            out[name] = upload(host[name], sdt, device)
        else:
            out[name] = S.gen.device_tensor(cfg, name, device)
    return out


def alloc_forward(cfg, device="cuda"):
    N, k = cfg.n_tokens, cfg.top_k
    dims = M.dims_of(cfg)
    ws = torch.empty(max(M.workspace_bytes(dims, M.ENTRY_FORWARD), 1), dtype=torch.uint8, device=device)
    return dict(
        dims=dims,
        y=torch.empty((N, cfg.d_model), dtype=torch_dtype(cfg.dtype), device=device),
        ids=torch.empty((N, k), dtype=torch.int32, device=device),
        probs=torch.empty((N, k), dtype=torch.float32, device=device),
        counts=torch.empty((cfg.n_routed,), dtype=torch.int32, device=device),
        ws=ws,
    )


def run_forward(cfg, dev_inputs: dict, bufs: dict) -> int:
    C = M.latentmoe_forward(bufs["dims"], dev_inputs, dev_inputs["x"], bufs["y"], bufs["ids"],
                            bufs["probs"], bufs["counts"], want_capacity=True, workspace=bufs["ws"])
    torch.cuda.synchronize()
    return C


def check_routes(gpu_ids: np.ndarray, routes, bias: np.ndarray, k: int) -> np.ndarray:
    """Near-tie rule.  Returns the mask of near-tie tokens.  Tokens with margin
    > MARGIN must select exactly the oracle's set; near-tie tokens must select
    a valid top-k of the oracle's s + b within MARGIN."""
    v = routes.s + bias[None, :]
    near = routes.margin <= MARGIN
    N, R = v.shape
    assert gpu_ids.shape == (N, k)
    assert ((gpu_ids >= 0) & (gpu_ids < R)).all()
    for n in range(N):
        assert len(set(gpu_ids[n].tolist())) == k, f"token {n}: repeated ids"
    far = ~near
    g_sorted = np.sort(gpu_ids[far], axis=1)
    o_sorted = np.sort(routes.ids[far], axis=1)
    bad = np.nonzero((g_sorted != o_sorted).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens routed differently with margin > {MARGIN}: {np.nonzero(far)[0][bad[:5]]}"
    for n in np.nonzero(near)[0]:
        vs = np.sort(v[n])[::-1]
        vk = vs[k - 1]
        vk1 = vs[k] if k < R else -np.inf
        chosen = np.zeros(R, bool)
        chosen[gpu_ids[n]] = True
        assert (v[n][chosen] >= vk - MARGIN).all()
        assert (v[n][~chosen] <= vk1 + MARGIN).all()
    return near


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))


TOL = {"f32": 1e-4, "bf16": 2e-2}
