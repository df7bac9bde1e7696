"""Helpers for the GPU tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np

from synth import inputs as S
from synth.configs import LayerConfig


def say(*a) -> None:
    """Name the case on stdout before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def torch_dtype(cfg: LayerConfig):
    import torch
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, cfg_dtype: str):
    """numpy (uint16 bf16 bits or float32/int32) -> torch CUDA tensor."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        assert cfg_dtype == "bf16"
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    """torch tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def values(a: np.ndarray) -> np.ndarray:
    """float64 values of a host array (bf16 bits widened)."""
    if a.dtype == np.uint16:
        return S.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def dims_of(moge, cfg: LayerConfig, T: int, M: int = None, kp: int = None):
    return moge.make_dims(T, cfg.d, cfg.N, cfg.M if M is None else M,
                          cfg.kp if kp is None else kp, cfg.inter, cfg.I_s,
                          moge.MOGE_BF16 if cfg.dtype == "bf16" else moge.MOGE_F32)


def normwise_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / max |ref| (the layer-output error measure)."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(y))) if y.size else 0.0
    return float(np.max(np.abs(y - ref))) / den


def tolerance(cfg: LayerConfig) -> float:
    return 2e-2 if cfg.dtype == "bf16" else 1e-5


@functools.lru_cache(maxsize=2)
def host_weights(key):
    cfg = key
    return S.make_weights(cfg)


def weight_key(cfg: LayerConfig) -> LayerConfig:
    """Configs that share every weight (same shapes, scales and seed) map to one key."""
    from dataclasses import replace
    return replace(cfg, name="weights", T=0, zipf_s=0.0, note="")


@functools.lru_cache(maxsize=2)
def device_weights(key):
    w = host_weights(key)
    return {k: (to_dev(v, key.dtype) if k != "router_bias" else None) for k, v in w.items()}


def layer_inputs(cfg: LayerConfig, T: int):
    """Host inputs and their device copies for one layer call (weights cached)."""
    k = weight_key(cfg)
    inp = S.make_layer_inputs(cfg, T=T, weights=host_weights(k))
    dw = dict(device_weights(k))
    dw["router_bias"] = to_dev(inp.router_bias, cfg.dtype) if inp.router_bias is not None else None
    dw["x"] = to_dev(inp.x, cfg.dtype)
    return inp, dw
