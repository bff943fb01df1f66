"""Host and device materialisation of the seeded inputs (see synth_core.h)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import TENSOR_IDS, LayerConfig, tensor_names, tensor_spec

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "liblmoe_synth_host.so")
DEV_LIB = os.path.join(_HERE, "liblmoe_synth_dev.so")

_host = None
_dev = None


def build_host() -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", HOST_LIB,
           os.path.join(_HERE, "synth_host.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return HOST_LIB


def build_device() -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", DEV_LIB, os.path.join(_HERE, "synth_dev.hip")]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return DEV_LIB


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        lib = ctypes.CDLL(HOST_LIB)
        i64, u64, u32, dbl, vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_double, ctypes.c_void_p)
        for fn in ("lmoe_synth_fill_normal_f32", "lmoe_synth_fill_normal_bf16"):
            getattr(lib, fn).argtypes = [vp, i64, i64, u64, u32, dbl, i64, i64, dbl]
            getattr(lib, fn).restype = None
        lib.lmoe_synth_fill_uniform_f32.argtypes = [vp, i64, i64, u64, u32, dbl, dbl]
        lib.lmoe_synth_fill_uniform_f32.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"device generator not built: {DEV_LIB} (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEV_LIB)
        i64, u64, u32, dbl, vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_double, ctypes.c_void_p)
        for fn in ("lmoe_synth_dev_fill_normal_f32", "lmoe_synth_dev_fill_normal_bf16"):
            getattr(lib, fn).argtypes = [vp, i64, i64, u64, u32, dbl, i64, i64, dbl, vp]
            getattr(lib, fn).restype = ctypes.c_int
        lib.lmoe_synth_dev_fill_uniform_f32.argtypes = [vp, i64, i64, u64, u32, dbl, dbl, vp]
        lib.lmoe_synth_dev_fill_uniform_f32.restype = ctypes.c_int
        _dev = lib
    return _dev


# ---------------------------------------------------------------- bf16 bits
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (fp32 array, or uint16 bf16 bits) -> exact fp64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- host side
def host_tensor(cfg: LayerConfig, name: str, start: int = 0, count: int | None = None) -> np.ndarray:
    """Flat slice [start, start+count) of one input tensor, as stored:
    float32 for fp32 tensors, uint16 bf16 bits for bf16 tensors."""
    shape, sdt, scale, row_len, rows_mult, row_mult = tensor_spec(cfg, name)
    total = int(np.prod(shape))
    if count is None:
        count = total - start
    if start < 0 or count < 0 or start + count > total:
        raise ValueError("slice out of range")
    if name == "rms_w":
        return np.ones(count, dtype=np.float32)
    if name == "bias":
        return _bias_host(cfg, start, count)
    lib = _host_lib()
    tid = TENSOR_IDS[name]
    if sdt == "bf16":
        out = np.empty(count, dtype=np.uint16)
        lib.lmoe_synth_fill_normal_bf16(out.ctypes.data, start, count, cfg.seed, tid, scale,
                                        row_len, rows_mult, row_mult)
    else:
        out = np.empty(count, dtype=np.float32)
        lib.lmoe_synth_fill_normal_f32(out.ctypes.data, start, count, cfg.seed, tid, scale,
                                       row_len, rows_mult, row_mult)
    return out


def _bias_host(cfg: LayerConfig, start: int, count: int) -> np.ndarray:
    R = cfg.n_routed
    if cfg.bias == "zero":
        b = np.zeros(R, dtype=np.float32)
    elif cfg.bias == "quadratic":
        i = np.arange(R, dtype=np.float64)
        b = (0.5 * (i / max(R - 1, 1)) ** 2).astype(np.float32)
    elif cfg.bias == "uniform":
        b = np.empty(R, dtype=np.float32)
        _host_lib().lmoe_synth_fill_uniform_f32(b.ctypes.data, 0, R, cfg.seed, TENSOR_IDS["bias"],
                                                -0.01, 0.01)
    else:
        raise ValueError(cfg.bias)
    return b[start:start + count].copy()


def host_inputs(cfg: LayerConfig) -> dict[str, np.ndarray]:
    """All inputs of a config on the host, shaped (stored dtype)."""
    out = {}
    for name in tensor_names(cfg):
        shape = tensor_spec(cfg, name)[0]
        out[name] = host_tensor(cfg, name).reshape(shape)
    return out


# -------------------------------------------------------------- device side
def device_tensor(cfg: LayerConfig, name: str, device="cuda"):
    """Materialise one input directly in device memory (torch tensor; bf16
    tensors as torch.bfloat16).  Same values as host_tensor."""
    import torch

    shape, sdt, scale, row_len, rows_mult, row_mult = tensor_spec(cfg, name)
    if name in ("bias", "rms_w"):
        return torch.from_numpy(host_tensor(cfg, name).reshape(shape)).to(device)
    tdt = torch.bfloat16 if sdt == "bf16" else torch.float32
    t = torch.empty(shape, dtype=tdt, device=device)
    n = t.numel()
    stream = torch.cuda.current_stream(t.device).cuda_stream
    lib = _dev_lib()
    fn = lib.lmoe_synth_dev_fill_normal_bf16 if sdt == "bf16" else lib.lmoe_synth_dev_fill_normal_f32
    rc = fn(t.data_ptr(), 0, n, cfg.seed, TENSOR_IDS[name], scale, row_len, rows_mult, row_mult, stream)
    if rc != 0:
        raise RuntimeError(f"device generator failed (hipError {rc}) for {name}")
    return t


def device_inputs(cfg: LayerConfig, device="cuda") -> dict:
    return {name: device_tensor(cfg, name, device) for name in tensor_names(cfg)}
