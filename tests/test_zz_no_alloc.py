"""The fixed-scratch forward (latentmoe_forward_noalloc, through the C ABI)
against the workspace forward (latentmoe_forward) on the same inputs: the
same kernels, so y, ids, probs and counts must be bit-identical.  Two calls
in a row share the device's scratch, the second with fewer tokens; the
range flag of the scratch is read through latentmoe_forward_check."""
import numpy as np
import pytest
import torch

import lmoe_synth as S
import mixture_experts_ffn_sigmoid_amd as M
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    M.load()


def _pair(cfg, dev):
    """Run both forms on cfg's first n_tokens rows of dev; return their outputs."""
    bufs = G.alloc_forward(cfg)
    W = M.weights_struct(dev)
    x = dev["x"][: cfg.n_tokens]
    M.latentmoe_forward(bufs["dims"], W, x, bufs["y"], bufs["ids"], bufs["probs"], bufs["counts"],
                        want_capacity=False, workspace=bufs["ws"])
    torch.cuda.synchronize()
    ref = {n: bufs[n].clone() for n in ("y", "ids", "probs", "counts")}
    nan = {n: torch.full_like(ref[n], -1) if ref[n].dtype == torch.int32 else torch.full_like(ref[n], float("nan"))
           for n in ref}
    M.latentmoe_forward_noalloc(bufs["dims"], W, x, nan["y"], nan["ids"], nan["probs"], nan["counts"])
    torch.cuda.synchronize()
    return ref, nan


@pytest.mark.parametrize("name,n1,n2", [("k3full_n64", 64, 9), ("b05skew_n4096", 4096, 1000), ("toy_n128", 128, 77)])
def test_noalloc_matches_workspace_forward_twice(name, n1, n2):
    base = S.CONFIGS[name]
    print(f"[noalloc] {name} N={n1} then N={n2}", flush=True)
    host = None if name.startswith("k3") else S.host_inputs(base)
    dev = G.device_layer_inputs(base, host=host)
    for n in (n1, n2):
        cfg = base.with_(n_tokens=n)
        ref, got = _pair(cfg, dev)
        for k in ref:
            a, b = ref[k], got[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (name, n, k)
        M.latentmoe_forward_check(M.dims_of(cfg), None)  # in range: no error
    print("   bit-identical on both calls", flush=True)


def test_noalloc_range_flag_is_readable():
    """x * 1e6 overflows z in fp16: the scratch's flag reports RANGE, and a
    following in-range call clears it."""
    cfg = S.CONFIGS["b05_n4096"].with_(n_tokens=512)
    host = dict(S.host_inputs(S.CONFIGS["b05_n4096"]))
    dev = G.device_layer_inputs(S.CONFIGS["b05_n4096"], host=host)
    xs = (dev["x"][:512].float() * 1e6).to(torch.bfloat16)
    bufs = G.alloc_forward(cfg)
    W = M.weights_struct(dev)
    M.latentmoe_forward_noalloc(bufs["dims"], W, xs, bufs["y"], bufs["ids"], bufs["probs"], bufs["counts"])
    with pytest.raises(M.LatentMoEError) as ei:
        M.latentmoe_forward_check(bufs["dims"], None)
    assert ei.value.status == 6
    M.latentmoe_forward_noalloc(bufs["dims"], W, dev["x"][:512], bufs["y"], bufs["ids"], bufs["probs"], bufs["counts"])
    M.latentmoe_forward_check(bufs["dims"], None)
