"""Seeded synthetic inputs for the MoGE layer (shared by the oracle tests, the
GPU tests and the benchmark).

This module draws random numbers and stores them in the layer's dtype.  It holds
none of the layer's arithmetic: no routing, no softmax, no matmul.

Recipe (every tensor):
  * values are float32 draws of standard_normal * std from numpy's PCG64;
  * a tensor is cut into chunks of CHUNK consecutive elements (row-major); chunk c
    of tensor `tid` is drawn from SeedSequence([seed, tid, c]), so the values do
    not depend on how many threads fill them;
  * bf16 tensors are rounded from those float32 values to nearest-even and kept
    as uint16 bit patterns (the upper half of the float32 word).

Tensor ids: 0 x[T,d], 1 w_router[N,d], 2 w_gate[N,I,d], 3 w_up[N,I,d],
4 w_down[N,d,I], 5 ws_gate[I_s,d], 6 ws_up[I_s,d], 7 ws_down[d,I_s],
8 router scores for the routing-only calls [T,N] (std 1),
20-25 int8 expert codes (gate, up, down, shared gate, shared up, shared down),
30-35 their per-row scales (same order).

int8 expert weights (the weight-only int8 layer): codes are float32 draws of
standard_normal * 32 with the chunked recipe above, rounded to the nearest integer
and clipped to [-127, 127]; per-row scales are (w_std / 32) * (1 + 0.25 u), u
uniform in [-1, 1) from SeedSequence([seed, tid]), so that scale * code has about
the spread of the bf16 weights.

Layouts are row-major with the contraction dimension contiguous for every weight:
a gate/up row is one intermediate unit's d inputs, a down row is one output
channel's I inputs.  The shared experts are stored concatenated along the
intermediate dimension: shared expert s owns rows [s*shared_inter,
(s+1)*shared_inter) of ws_gate/ws_up and the same columns of ws_down.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import LayerConfig

CHUNK = 1 << 20

TID_X, TID_WR, TID_WG, TID_WU, TID_WD, TID_WSG, TID_WSU, TID_WSD, TID_SCORES = range(9)
TID_QG, TID_QU, TID_QD, TID_QSG, TID_QSU, TID_QSD = range(20, 26)
TID_SG, TID_SU, TID_SD, TID_SSG, TID_SSU, TID_SSD = range(30, 36)
CODE_STD = 32.0


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_tensor(shape, std: float, seed: int, tid: int, dtype: str) -> np.ndarray:
    """Draw a tensor of N(0, std) values with the chunked recipe above.

    dtype "f32" returns float32, "bf16" returns uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    s32 = np.float32(std)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        v *= s32
        if dtype == "bf16":
            out[lo:hi] = f32_to_bf16_bits(v)
        else:
            out[lo:hi] = v

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def zipf_bias(N: int, s: float) -> np.ndarray:
    """Per-expert router bias -s*ln(rank) with rank = e+1 (float32).

    Adding it to the router scores makes the scores of expert e follow a
    Zipf(s)-shaped preference: low-numbered experts are favoured, so a plain global
    top-K overloads the first groups."""
    return (-np.float32(s) * np.log(np.arange(1, N + 1, dtype=np.float64))).astype(np.float32)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray                 # [T,d]
    w_router: np.ndarray          # [N,d]
    router_bias: Optional[np.ndarray]  # [N] float32 or None
    w_gate: np.ndarray            # [N,I,d]
    w_up: np.ndarray              # [N,I,d]
    w_down: np.ndarray            # [N,d,I]
    ws_gate: np.ndarray           # [I_s,d]
    ws_up: np.ndarray             # [I_s,d]
    ws_down: np.ndarray           # [d,I_s]

    @property
    def is_bf16(self) -> bool:
        return self.cfg.dtype == "bf16"


def make_weights(cfg: LayerConfig, seed: Optional[int] = None) -> dict:
    """The layer's weights (they do not depend on T)."""
    seed = cfg.seed if seed is None else seed
    dt = cfg.dtype
    d, N, I, Is = cfg.d, cfg.N, cfg.inter, cfg.I_s
    return dict(
        w_router=normal_tensor((N, d), cfg.router_std, seed, TID_WR, dt),
        router_bias=zipf_bias(N, cfg.zipf_s) if cfg.zipf_s > 0 else None,
        w_gate=normal_tensor((N, I, d), cfg.w_std, seed, TID_WG, dt),
        w_up=normal_tensor((N, I, d), cfg.w_std, seed, TID_WU, dt),
        w_down=normal_tensor((N, d, I), cfg.w_std, seed, TID_WD, dt),
        ws_gate=normal_tensor((Is, d), cfg.w_std, seed, TID_WSG, dt),
        ws_up=normal_tensor((Is, d), cfg.w_std, seed, TID_WSU, dt),
        ws_down=normal_tensor((d, Is), cfg.w_std, seed, TID_WSD, dt),
    )


def int8_codes(shape, seed: int, tid: int) -> np.ndarray:
    """Seeded int8 codes: rint(standard_normal * 32) clipped to [-127, 127]."""
    v = normal_tensor(shape, CODE_STD, seed, tid, "f32")
    return np.clip(np.rint(v), -127, 127).astype(np.int8)


def row_scales(n: int, mean: float, seed: int, tid: int) -> np.ndarray:
    """Seeded per-row scales mean * (1 + 0.25 u), u ~ U[-1, 1), float32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))
    u = g.random(n, dtype=np.float64) * 2.0 - 1.0
    return (mean * (1.0 + 0.25 * u)).astype(np.float32)


def make_w8_weights(cfg: LayerConfig, seed: Optional[int] = None) -> dict:
    """int8 codes and float32 per-row scales of the expert and shared weights
    (shapes of make_weights; scales [.., rows]).  The router keeps make_weights'
    bf16 w_router."""
    seed = cfg.seed if seed is None else seed
    d, N, I, Is = cfg.d, cfg.N, cfg.inter, cfg.I_s
    m = cfg.w_std / CODE_STD
    return dict(
        q_gate=int8_codes((N, I, d), seed, TID_QG), s_gate=row_scales(N * I, m, seed, TID_SG).reshape(N, I),
        q_up=int8_codes((N, I, d), seed, TID_QU), s_up=row_scales(N * I, m, seed, TID_SU).reshape(N, I),
        q_down=int8_codes((N, d, I), seed, TID_QD), s_down=row_scales(N * d, m, seed, TID_SD).reshape(N, d),
        qs_gate=int8_codes((Is, d), seed, TID_QSG), ss_gate=row_scales(Is, m, seed, TID_SSG),
        qs_up=int8_codes((Is, d), seed, TID_QSU), ss_up=row_scales(Is, m, seed, TID_SSU),
        qs_down=int8_codes((d, Is), seed, TID_QSD), ss_down=row_scales(d, m, seed, TID_SSD),
    )


def make_x(cfg: LayerConfig, T: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    """Activations x[T,d]; row t does not depend on T (drawn row-major)."""
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    return normal_tensor((T, cfg.d), cfg.x_std, seed, TID_X, cfg.dtype)


def make_layer_inputs(cfg: LayerConfig, T: Optional[int] = None,
                      seed: Optional[int] = None, weights: Optional[dict] = None) -> LayerInputs:
    """All tensors of one layer call, seeded.  T overrides cfg.T.  `weights` may
    pass in a make_weights() result to avoid drawing the weights again."""
    w = make_weights(cfg, seed) if weights is None else weights
    if cfg.zipf_s > 0:
        w = dict(w, router_bias=zipf_bias(cfg.N, cfg.zipf_s))
    else:
        w = dict(w, router_bias=None)
    return LayerInputs(cfg=cfg, x=make_x(cfg, T, seed), **w)


def make_scores(cfg: LayerConfig, T: Optional[int] = None, seed: Optional[int] = None,
                with_bias: bool = True) -> np.ndarray:
    """Router scores [T,N] float32 ~ N(0,1) for the routing-only calls, plus the
    Zipf bias when the workload has one.  These set the per-expert row counts of
    the routing/permutation workloads."""
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    s = normal_tensor((T, cfg.N), 1.0, seed, TID_SCORES, "f32")
    if with_bias and cfg.zipf_s > 0:
        s = (s + zipf_bias(cfg.N, cfg.zipf_s)[None, :]).astype(np.float32)
    return s


def tie_scores(T: int, N: int, seed: int, levels: int = 3) -> np.ndarray:
    """Scores with many exact ties (small integers, with +0.0 and -0.0 both
    present) for the tie-breaking cases."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    v = g.integers(-levels, levels + 1, size=(T, N)).astype(np.float32)
    neg0 = g.random((T, N)) < 0.5
    v[(v == 0) & neg0] = np.float32(-0.0)
    return v


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """A sorted seeded sample of n distinct token indices (all tokens if n >= T);
    always includes the first and last token."""
    if n >= T:
        return np.arange(T)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    pick = g.choice(np.arange(1, T - 1), size=max(0, n - 2), replace=False)
    return np.unique(np.concatenate([[0, T - 1], pick])).astype(np.int64)
