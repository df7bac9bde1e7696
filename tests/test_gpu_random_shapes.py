"""Seeded random layer shapes through the C ABI, against the oracle.

Each case draws a layer (fp32 or bf16; N, M, K', widths that do and do not fit the
MFMA tile shapes; with and without shared experts and router bias) and a batch
size, runs the row-major, packed and (where its sizes allow) int8 layers on given
router scores, and checks: routing bit-exact, packed == row-major bit for bit,
outputs within the layer tolerance of the oracle."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moge_oracle as O
from synth import inputs as S
from synth.configs import C0
from tests.gpu_util import (dims_of, normwise_rel_err, say, to_dev, to_host, tolerance,
                            values)


def _draw(seed):
    if (seed // 16) % 2:
        return _draw_tiles(seed)
    rng = np.random.Generator(np.random.PCG64([2024, seed]))
    dtype = ["f32", "bf16"][seed % 2]
    d = int(rng.choice([64, 128, 256, 512]))
    N = int(rng.choice([8, 16, 32, 64]))
    M = int(rng.choice([m for m in (1, 2, 4, 8) if N % m == 0]))
    kp = int(rng.integers(1, min(N // M, 64 // M, 3) + 1))
    inter = int(rng.choice([32, 64, 96, 128, 192]))
    n_sh = int(rng.choice([0, 1, 2]))
    sh_w = int(rng.choice([64, 96]))
    T = int(rng.choice([1, 7, 33, 64, 100, 200, 300]))
    zipf = float(rng.choice([0.0, 1.2]))
    cfg = replace(C0, name=f"random-{seed}", T=T, d=d, N=N, M=M, kp=kp, inter=inter,
                  n_shared=n_sh, shared_inter=sh_w if n_sh else 0, dtype=dtype,
                  router_std=1.0 / np.sqrt(d), zipf_s=zipf, seed=seed)
    return cfg


def _draw_tiles(seed):
    """bf16 layers whose widths fit the MFMA tile shapes (multiples of 192), with
    batches whose experts reach the 64-row and 256-row tiles"""
    rng = np.random.Generator(np.random.PCG64([2025, seed]))
    d = int(rng.choice([256, 512]))
    N = int(rng.choice([8, 16]))
    M = int(rng.choice([m for m in (2, 4, 8) if N % m == 0]))
    kp = int(rng.integers(1, min(N // M, 2) + 1))
    inter = int(rng.choice([192, 384]))
    n_sh = int(rng.choice([0, 1, 2]))
    T = int(rng.choice([100, 300, 600]))
    return replace(C0, name=f"random-tiles-{seed}", T=T, d=d, N=N, M=M, kp=kp, inter=inter,
                   n_shared=n_sh, shared_inter=192 if n_sh else 0, dtype="bf16",
                   router_std=1.0 / np.sqrt(d), zipf_s=float(rng.choice([0.0, 1.2])), seed=seed)


# seeds 0-15 and 32-47: any shape; 16-31 and 48-63: shapes and batches for the
# tile kernels
CASES = list(range(64))

# Skewed batches (Zipf(1.2) router bias) at the edges of the host's row-range
# choice, which uses only the mean rows per expert R / N:
#   mean 50 (T=400, N=64, K=8): no streaming launch, no 256-row launch, so the
#     64-row tiles take experts of any size, from a few rows to several hundred;
#     the shared segment runs beside them on 256-row tiles (one full, one partial),
#     its down contraction whole (width 192: 3 stages) or in two slices (two
#     experts of 384, width 768: 12 stages);
#   mean 512 (T=2048, N=16, K=4): every routed expert on 256-row tiles, the
#     least-chosen ones with far fewer than 128 rows.
EDGE_CASES = {
    "mean50-skewed": replace(C0, name="mean50-skewed", T=400, d=256, N=64, M=8, kp=1, inter=192,
                             n_shared=1, shared_inter=192, dtype="bf16", router_std=1.0 / 16,
                             zipf_s=1.2, seed=7),
    "mean50-sliced-shared": replace(C0, name="mean50-sliced-shared", T=400, d=256, N=64, M=8,
                                    kp=1, inter=192, n_shared=2, shared_inter=384,
                                    dtype="bf16", router_std=1.0 / 16, zipf_s=1.2, seed=9),
    "mean512-skewed": replace(C0, name="mean512-skewed", T=2048, d=256, N=16, M=4, kp=1,
                              inter=192, n_shared=1, shared_inter=192, dtype="bf16",
                              router_std=1.0 / 16, zipf_s=1.2, seed=8),
}

# The API's limits: N = 256 experts and K = M * K' = 64 slots per token (4 groups of
# 64, 16 from each).  T = 1 (64 experts with one row each), T = 100 (mean 25 rows:
# streaming and 64-row tiles), T = 600 (mean 150: 64-row and 256-row tiles).
LIMIT_CASES = [(dt, T) for dt in ("bf16", "f32") for T in (1, 100, 600)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,T", LIMIT_CASES)
def test_layer_at_api_limits(lib, dtype, T):
    cfg = replace(C0, name=f"limits-{dtype}-T{T}", T=T, d=256, N=256, M=4, kp=16, inter=192,
                  n_shared=1, shared_inter=192, dtype=dtype, router_std=1.0 / 16, zipf_s=0.0,
                  seed=11)
    # T = 600: the oracle's float64 layer over 38400 rows takes about a minute, so
    # its outputs are compared on 64 sampled tokens (routing on all of them)
    _check_layer(lib, cfg, tokens=S.sample_tokens(T, 64) if T > 100 else None)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", CASES)
def test_random_layer(lib, seed):
    _check_layer(lib, _draw(seed))


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_row_range_edges(lib, name):
    cfg = EDGE_CASES[name]
    counts = np.bincount(O.route(S.make_scores(cfg, T=cfg.T), cfg.M, cfg.kp)["idx"].ravel(),
                         minlength=cfg.N)
    # the shapes reach what they are for
    if name.startswith("mean50"):
        assert counts.max() > 128 and counts.min() <= 32, counts
    else:
        assert counts.min() < 128, counts
    _check_layer(lib, cfg)


def _check_layer(lib, cfg, tokens=None):
    import torch
    seed = cfg.seed
    T = cfg.T
    inp = S.make_layer_inputs(cfg)
    scores = S.make_scores(cfg, T=T)
    dims = dims_of(lib, cfg, T)
    dt = cfg.dtype
    dev = {k: to_dev(getattr(inp, k), dt) for k in ("x", "w_gate", "w_up", "w_down")}
    shared = cfg.I_s > 0
    for k in ("ws_gate", "ws_up", "ws_down"):
        dev[k] = to_dev(getattr(inp, k), dt) if shared else None
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ws = torch.empty(lib.workspace_size(dims), dtype=torch.uint8, device="cuda")
    lin = to_dev(scores, "f32")
    say("random layer", seed, cfg)

    def outs():
        return (torch.empty((T, cfg.d), dtype=tdt, device="cuda"),
                torch.empty((T, dims.K), dtype=torch.int32, device="cuda"))

    y, idx = outs()
    lib.layer_forward(dims, dev["x"], None, None, dev["w_gate"], dev["w_up"], dev["w_down"],
                      dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws, logits_in=lin,
                      topk_idx_out=idx)
    packed = torch.empty(lib.packed_weights_size(dims), dtype=torch.uint8, device="cuda")
    lib.pack_weights(dims, dev["w_gate"], dev["w_up"], dev["w_down"], dev["ws_gate"],
                     dev["ws_up"], dev["ws_down"], packed)
    yp, idxp = outs()
    lib.layer_forward_packed(dims, dev["x"], None, None, packed, yp, ws, logits_in=lin,
                             topk_idx_out=idxp)
    torch.cuda.synchronize()
    ref = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  inp.ws_gate, inp.ws_up, inp.ws_down, M=cfg.M, kp=cfg.kp, dtype=dt,
                  logits_f32=scores, tokens=tokens)
    rows = slice(None) if tokens is None else tokens
    np.testing.assert_array_equal(to_host(idx), ref["idx"])
    np.testing.assert_array_equal(to_host(idxp), ref["idx"])
    np.testing.assert_array_equal(to_host(yp), to_host(y))
    err = normwise_rel_err(values(to_host(y))[rows], ref["y"])
    assert err <= tolerance(cfg), err

    # the int8 layer where the sizes allow it (bf16, widths multiples of 64)
    w8_ok = dt == "bf16" and cfg.d % 64 == 0 and cfg.inter % 64 == 0 and cfg.I_s % 64 == 0
    assert (lib.w8_weights_size(dims) > 0) == w8_ok
    if not w8_ok:
        return
    buf = torch.empty(lib.w8_weights_size(dims), dtype=torch.uint8, device="cuda")
    lib.quantize_weights_w8(dims, dev["w_gate"], dev["w_up"], dev["w_down"], dev["ws_gate"],
                            dev["ws_up"], dev["ws_down"], buf)
    y8, idx8 = outs()
    lib.layer_forward_w8(dims, dev["x"], None, None, buf, y8, ws, logits_in=lin,
                         topk_idx_out=idx8)
    torch.cuda.synchronize()
    q = {}
    for key, skey, src in (("q_gate", "s_gate", inp.w_gate), ("q_up", "s_up", inp.w_up),
                           ("q_down", "s_down", inp.w_down)):
        q[key], q[skey] = O.w8_quantize(src, "bf16")
    if shared:
        for key, skey, src in (("qs_gate", "ss_gate", inp.ws_gate), ("qs_up", "ss_up", inp.ws_up),
                               ("qs_down", "ss_down", inp.ws_down)):
            q[key], q[skey] = O.w8_quantize(src, "bf16")
        ref8 = O.layer_w8(inp.x, inp.w_router, inp.router_bias, q["q_gate"], q["s_gate"],
                          q["q_up"], q["s_up"], q["q_down"], q["s_down"], q["qs_gate"],
                          q["ss_gate"], q["qs_up"], q["ss_up"], q["qs_down"], q["ss_down"],
                          M=cfg.M, kp=cfg.kp, logits_f32=scores, tokens=tokens)
    else:
        # no shared experts: the int8 layer of the routed experts alone
        ref8 = O.layer(inp.x, inp.w_router, inp.router_bias, O.W8Weights(q["q_gate"], q["s_gate"]),
                       O.W8Weights(q["q_up"], q["s_up"]), O.W8Weights(q["q_down"], q["s_down"]),
                       np.zeros((0, cfg.d)), np.zeros((0, cfg.d)), np.zeros((cfg.d, 0)),
                       M=cfg.M, kp=cfg.kp, dtype="bf16", logits_f32=scores, wdtype="f64",
                       tokens=tokens)
    np.testing.assert_array_equal(to_host(idx8), ref["idx"])
    err8 = normwise_rel_err(values(to_host(y8))[rows], ref8["y"])
    assert err8 <= tolerance(cfg), err8
