"""GPU parity: every entry point of the C ABI against the CPU oracle on the same
seeded inputs.  Routing and permutation must match bit for bit; float outputs
within max|y - ref| / max|ref| <= 2e-2 (bf16 storage, fp32 accumulation) or
1e-5 (fp32 configuration)."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moge_oracle as O
from synth import inputs as S
from synth.configs import C0, C1, C2, C3, C4, CONFIGS
from tests.gpu_util import (dims_of, layer_inputs, normwise_rel_err, say, to_dev, to_host,
                            tolerance, values)

pytestmark = pytest.mark.gpu

ALL = ["C0", "C1", "C2", "C3", "C4"]


def _empty(shape, dt):
    import torch
    return torch.empty(shape, dtype=dt, device="cuda")


def _route_gpu(moge, cfg, scores, M=None, kp=None):
    import torch
    T = scores.shape[0]
    dims = dims_of(moge, cfg, T, M, kp)
    idx = _empty((T, dims.K), torch.int32)
    gate = _empty((T, dims.K), torch.float32)
    probs = _empty((T, cfg.N), torch.float32)
    moge.route(dims, to_dev(scores, "f32"), idx, gate, probs)
    torch.cuda.synchronize()
    return to_host(idx), to_host(gate), to_host(probs)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ALL)
def test_route_bit_exact(lib, name):
    cfg = CONFIGS[name]
    scores = S.make_scores(cfg)
    say("route", name, scores.shape)
    idx, gate, probs = _route_gpu(lib, cfg, scores)
    r = O.route(scores, cfg.M, cfg.kp)
    np.testing.assert_array_equal(idx, r["idx"])
    assert np.max(np.abs(gate - r["gate"])) <= 1e-6
    assert np.max(np.abs(probs - r["probs"])) <= 1e-6
    np.testing.assert_allclose(probs.astype(np.float64).sum(1), 1.0, atol=1e-5)


@pytest.mark.parametrize("N,M,kp", [(8, 2, 1), (8, 2, 2), (16, 4, 1), (64, 8, 1), (64, 8, 2),
                                    (64, 1, 8), (256, 8, 4), (12, 3, 2), (64, 64, 1),
                                    (256, 4, 16), (96, 2, 32)])
def test_route_ties_and_shapes(lib, N, M, kp):
    cfg = replace(C0, N=N, M=M, kp=kp)
    scores = S.tie_scores(203, N, seed=N * 7 + M + kp)
    say("route ties", N, M, kp)
    idx, gate, _ = _route_gpu(lib, cfg, scores)
    r = O.route(scores, M, kp)
    np.testing.assert_array_equal(idx, r["idx"])
    assert np.max(np.abs(gate - r["gate"])) <= 1e-6


def test_route_all_equal_scores(lib):
    cfg = C1
    for val in (0.0, -0.0, 3.5):
        scores = np.full((70, 64), val, dtype=np.float32)
        say("route all-equal", val)
        idx, gate, _ = _route_gpu(lib, cfg, scores)
        np.testing.assert_array_equal(idx, np.tile(np.arange(0, 64, 8, dtype=np.int32), (70, 1)))
        np.testing.assert_allclose(gate, 1 / 64, rtol=1e-6)


def test_global_topk_imbalance_vs_moge(lib):
    # the conventional router (one group, K=8) on the Zipf-biased scores overloads
    # the first groups; the grouped router's loads are all equal
    cfg = C4
    scores = S.make_scores(cfg)
    say("global top-8 vs MoGE", scores.shape)
    gidx, _, _ = _route_gpu(lib, cfg, scores, M=1, kp=8)
    np.testing.assert_array_equal(gidx, O.global_topk(scores, 8))
    loads = O.group_loads_of(gidx, 64, 8)
    assert O.imbalance_score(loads, cfg.T) > 1.0
    midx, _, _ = _route_gpu(lib, cfg, scores)
    assert O.imbalance_score(O.group_loads_of(midx, 64, 8), cfg.T) == 0.0


# ----------------------------------------------------------------------------
# permutation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("C0", 64), ("C1", 64), ("C2", 456), ("C3", 4096),
                                    ("C4", 16384), ("C1", 1), ("C1", 65), ("C0", 127)])
def test_permute_bit_exact(lib, name, T):
    import torch
    cfg = CONFIGS[name]
    scores = S.make_scores(cfg, T=T)
    idx = O.route(scores, cfg.M, cfg.kp)["idx"]
    ref = O.permute(idx, cfg.N, cfg.M)
    dims = dims_of(lib, cfg, T)
    x = to_dev(S.make_x(cfg, T), cfg.dtype)
    out = {k: _empty(n, torch.int32) for k, n in
           (("counts", cfg.N), ("offsets", cfg.N + 1), ("group_counts", cfg.M),
            ("sorted_pair", dims.R), ("pair_row", dims.R))}
    x_perm = _empty((dims.R, cfg.d), x.dtype)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    say("permute", name, T)
    lib.permute(dims, to_dev(idx, "f32"), x, out["counts"], out["offsets"], out["group_counts"],
                out["sorted_pair"], out["pair_row"], x_perm, ws)
    torch.cuda.synchronize()
    for k in out:
        np.testing.assert_array_equal(to_host(out[k]), ref[k], err_msg=k)
    assert (to_host(out["group_counts"]) == T * cfg.kp).all()
    src = torch.from_numpy(ref["sorted_pair"].astype(np.int64) // dims.K).cuda()
    assert torch.equal(x_perm, x.index_select(0, src))


@pytest.mark.parametrize("T", [64, 300, 512, 513, 2000])
def test_permute_arbitrary_choices(lib, T):
    # K distinct experts per token, not one per group and heavily skewed (expert 0
    # in most tokens): uneven counts and group loads; 512/513 straddle the switch
    # from the single-workgroup kernel to the chunk-parallel ones
    import torch
    cfg = C1
    rng = np.random.Generator(np.random.PCG64(T))
    w = 1.0 / np.arange(1, cfg.N + 1) ** 1.5
    idx = np.stack([rng.choice(cfg.N, size=cfg.K, replace=False, p=w / w.sum())
                    for _ in range(T)]).astype(np.int32)
    ref = O.permute(idx, cfg.N, cfg.M)
    dims = dims_of(lib, cfg, T)
    out = {k: _empty(n, torch.int32) for k, n in
           (("counts", cfg.N), ("offsets", cfg.N + 1), ("group_counts", cfg.M),
            ("sorted_pair", dims.R), ("pair_row", dims.R))}
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    say("permute arbitrary", T)
    lib.permute(dims, to_dev(idx, "f32"), None, out["counts"], out["offsets"],
                out["group_counts"], out["sorted_pair"], out["pair_row"], None, ws)
    torch.cuda.synchronize()
    for k in out:
        np.testing.assert_array_equal(to_host(out[k]), ref[k], err_msg=k)
    assert ref["counts"][0] > T // 2


# ----------------------------------------------------------------------------
# expert FFN (step API) and shared experts through the same entry point
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("C0", 64), ("C1", 64), ("C2", 456), ("C0", 37)])
def test_expert_ffn(lib, name, T):
    import torch
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    idx = O.route(scores, cfg.M, cfg.kp)["idx"]
    perm = O.permute(idx, cfg.N, cfg.M)
    dims = dims_of(lib, cfg, T)
    x_perm_h = inp.x[perm["sorted_pair"].astype(np.int64) // dims.K]
    y_perm = _empty((dims.R, cfg.d), dw["x"].dtype)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    say("expert_ffn", name, T)
    lib.expert_ffn(dims, to_dev(x_perm_h, cfg.dtype), to_dev(perm["offsets"], "f32"),
                   dw["w_gate"], dw["w_up"], dw["w_down"], y_perm, ws)
    torch.cuda.synchronize()
    ref = O.expert_ffn(O.to_f64(x_perm_h, cfg.dtype), perm["offsets"], inp.w_gate, inp.w_up,
                       inp.w_down, cfg.dtype)
    err = normwise_rel_err(values(to_host(y_perm)), ref)
    assert err <= tolerance(cfg), err


# Per-expert row counts on both sides of the switch between the streaming kernels
# (up to 32 rows) and the 64-row tiles, with partial tiles of every kind.  At a
# mean under 64 rows per expert the experts of more than 128 rows take 64-row
# tiles as well; the 256-row tiles are covered below.  The oracle checks sampled
# rows of every expert.
BOUNDARY_ROWS = [0, 1, 16, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 513]


def test_expert_ffn_row_count_boundaries(lib):
    import torch
    cfg = C1
    rows = list(BOUNDARY_ROWS)
    rows += [0] * (cfg.N - len(rows))
    rows[-1] = (-sum(rows)) % cfg.K            # total divisible by K
    counts = np.array(rows, dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    T = R // cfg.K
    inp, dw = layer_inputs(cfg, 64)            # weights only
    x_perm_h = S.make_x(cfg, T=R, seed=7)
    dims = dims_of(lib, cfg, T)
    y_perm = _empty((R, cfg.d), dw["x"].dtype)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    say("expert_ffn boundaries", R)
    lib.expert_ffn(dims, to_dev(x_perm_h, cfg.dtype), to_dev(offsets, "f32"),
                   dw["w_gate"], dw["w_up"], dw["w_down"], y_perm, ws)
    torch.cuda.synchronize()
    y = values(to_host(y_perm))
    # sampled rows of every expert: first, last, and two inside
    pick, sub_counts = [], []
    for e in range(cfg.N):
        lo, c = int(offsets[e]), int(counts[e])
        sel = sorted({lo + j for j in (0, c // 3, (2 * c) // 3, c - 1) if 0 <= j < c})
        pick += sel
        sub_counts.append(len(sel))
    pick = np.array(pick, dtype=np.int64)
    sub_off = np.concatenate([[0], np.cumsum(sub_counts)]).astype(np.int64)
    ref = O.expert_ffn(O.to_f64(x_perm_h[pick], cfg.dtype), sub_off, inp.w_gate, inp.w_up,
                       inp.w_down, cfg.dtype)
    err = normwise_rel_err(y[pick], ref)
    assert err <= tolerance(cfg), err


# Experts of more than 128 rows on 256-row tiles (a mean of 64-256 rows per expert
# keeps both tile launches), with last row tiles that leave each wave's four
# 32-row blocks full, partly filled or empty; experts of up to 128 rows on 64-row
# tiles beside them.  Every 32-row block boundary of each expert's last 288 rows
# is sampled.
PARTIAL_TILE_ROWS = [129, 160, 255, 256, 257, 263, 287, 288, 289, 319, 320, 352, 383, 384,
                     385, 416, 448, 449, 480, 511, 512, 513, 600, 769,
                     0, 1, 33, 64, 65, 100, 128]


def test_expert_ffn_partial_256_row_tiles(lib):
    import torch
    cfg = C1
    rows = list(PARTIAL_TILE_ROWS) + [150] * (cfg.N - len(PARTIAL_TILE_ROWS))
    rows[-1] += (-sum(rows)) % cfg.K           # total divisible by K
    counts = np.array(rows, dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    assert 64 < R / cfg.N < 256
    T = R // cfg.K
    inp, dw = layer_inputs(cfg, 64)            # weights only
    x_perm_h = S.make_x(cfg, T=R, seed=8)
    dims = dims_of(lib, cfg, T)
    y_perm = _empty((R, cfg.d), dw["x"].dtype)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    say("expert_ffn partial 256-row tiles", R)
    lib.expert_ffn(dims, to_dev(x_perm_h, cfg.dtype), to_dev(offsets, "f32"),
                   dw["w_gate"], dw["w_up"], dw["w_down"], y_perm, ws)
    torch.cuda.synchronize()
    y = values(to_host(y_perm))
    pick, sub_counts = [], []
    for e in range(cfg.N):
        lo, c = int(offsets[e]), int(counts[e])
        sel = {j for j in (0, c // 2, c - 1) if 0 <= j < c}
        sel |= {j for j in range(max(0, c - 288), c) if j % 32 in (0, 31)}
        pick += sorted(lo + j for j in sel)
        sub_counts.append(len(sel))
    pick = np.array(pick, dtype=np.int64)
    sub_off = np.concatenate([[0], np.cumsum(sub_counts)]).astype(np.int64)
    ref = O.expert_ffn(O.to_f64(x_perm_h[pick], cfg.dtype), sub_off, inp.w_gate, inp.w_up,
                       inp.w_down, cfg.dtype)
    err = normwise_rel_err(y[pick], ref)
    assert err <= tolerance(cfg), err
    # and no row of any expert is left unwritten or non-finite
    assert np.isfinite(y).all()


@pytest.mark.parametrize("name,T", [("C0", 64), ("C1", 64), ("C1", 100)])
def test_shared_expert_via_expert_ffn(lib, name, T):
    import torch
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    dims = lib.make_dims(T, cfg.d, 1, 1, 1, cfg.I_s, 0, dims_of(lib, cfg, T).dtype)
    y = _empty((T, cfg.d), dw["x"].dtype)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    say("shared via expert_ffn", name, T)
    lib.expert_ffn(dims, dw["x"], to_dev(np.array([0, T], dtype=np.int32), "f32"),
                   dw["ws_gate"], dw["ws_up"], dw["ws_down"], y, ws)
    torch.cuda.synchronize()
    ref = O.shared_experts(O.to_f64(inp.x, cfg.dtype), inp.ws_gate, inp.ws_up, inp.ws_down,
                           cfg.dtype)
    assert normwise_rel_err(values(to_host(y)), ref) <= tolerance(cfg)


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,T,with_shared", [("C0", 64, True), ("C1", 64, True),
                                                ("C1", 33, False)])
def test_combine(lib, name, T, with_shared):
    import torch
    cfg = CONFIGS[name]
    scores = S.make_scores(cfg, T=T)
    r = O.route(scores, cfg.M, cfg.kp)
    perm = O.permute(r["idx"], cfg.N, cfg.M)
    dims = dims_of(lib, cfg, T)
    y_perm = S.normal_tensor((dims.R, cfg.d), 1.0, 5, 20, cfg.dtype)
    sh = S.normal_tensor((T, cfg.d), 1.0, 5, 21, cfg.dtype) if with_shared else None
    y = _empty((T, cfg.d), torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    say("combine", name, T, with_shared)
    lib.combine(dims, to_dev(y_perm, cfg.dtype), to_dev(perm["pair_row"], "f32"),
                to_dev(r["gate"].astype(np.float32), "f32"),
                to_dev(sh, cfg.dtype) if sh is not None else None, y)
    torch.cuda.synchronize()
    ref = O.combine(O.to_f64(y_perm, cfg.dtype), perm["pair_row"], r["gate"].astype(np.float32),
                    O.to_f64(sh, cfg.dtype) if sh is not None else None, T, dims.K)
    tol = 2 ** -8 if cfg.dtype == "bf16" else 1e-6    # one final rounding
    assert normwise_rel_err(values(to_host(y)), ref) <= tol


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def _run_layer(lib, cfg, T, dw, logits_in=None):
    import torch
    dims = dims_of(lib, cfg, T)
    out = dict(y=_empty((T, cfg.d), dw["x"].dtype),
               logits=_empty((T, cfg.N), torch.float32),
               idx=_empty((T, dims.K), torch.int32),
               gate=_empty((T, dims.K), torch.float32),
               gc=_empty((cfg.M,), torch.int32))
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    lib.layer_forward(dims, dw["x"], dw["w_router"], dw["router_bias"], dw["w_gate"], dw["w_up"],
                      dw["w_down"], dw["ws_gate"], dw["ws_up"], dw["ws_down"], out["y"], ws,
                      logits_in=None if logits_in is None else to_dev(logits_in, "f32"),
                      logits_out=out["logits"], topk_idx_out=out["idx"],
                      topk_gate_out=out["gate"], group_counts_out=out["gc"])
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _sample(T):
    return S.sample_tokens(T, 48)


@pytest.mark.parametrize("name,T", [("C0", 64), ("C1", 64), ("C2", 456), ("C3", 4096),
                                    ("C4", 16384), ("C0", 1), ("C0", 65), ("C1", 17),
                                    # the shared segment's switches: streaming up to 64
                                    # rows, 64-row tiles up to 128 (gate/up) / 512 (down)
                                    ("C1", 65), ("C1", 128), ("C1", 129), ("C1", 512),
                                    ("C1", 513)])
def test_layer_on_given_scores(lib, name, T):
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    say("layer (given scores)", name, T)
    out = _run_layer(lib, cfg, T, dw, logits_in=scores)
    r = O.route(scores, cfg.M, cfg.kp)
    np.testing.assert_array_equal(out["idx"], r["idx"])
    assert (out["gc"] == T * cfg.kp).all()
    np.testing.assert_array_equal(out["logits"], scores)
    tok = _sample(T)
    ref = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  inp.ws_gate, inp.ws_up, inp.ws_down, M=cfg.M, kp=cfg.kp, dtype=cfg.dtype,
                  logits_f32=scores, tokens=tok)
    err = normwise_rel_err(values(out["y"])[tok], ref["y"])
    assert err <= tolerance(cfg), err


# Small bf16 layers that reach code paths the full-size workloads do not:
#  SB1: shapes the tile kernels do not cover (widths not a multiple of 96), so the
#       streaming kernels take every expert, in several 64-row passes;
#  SB2: tile shapes with contractions shorter than the LDS rings (gate/up 4
#       stages of 64, down 3 routed and 6 shared), at batch sizes that send the
#       experts to the streaming kernels (T=16), to 64-row tiles (T=300: about 75
#       rows per expert; the 300-row shared segment takes 256-row tiles for gate/up
#       and 64-row tiles for down) and to 256-row tiles (T=1200).
SB1 = replace(C0, name="SB1-bf16-streaming-only", dtype="bf16")
SB2 = replace(C0, name="SB2-bf16-short-contractions", dtype="bf16", inter=192, shared_inter=384)


@pytest.mark.parametrize("cfg,T", [(SB1, 300), (SB2, 16), (SB2, 300), (SB2, 1200)])
def test_small_bf16_layers(lib, cfg, T):
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    say("small bf16 layer", cfg.name, T)
    out = _run_layer(lib, cfg, T, dw, logits_in=scores)
    r = O.route(scores, cfg.M, cfg.kp)
    np.testing.assert_array_equal(out["idx"], r["idx"])
    tok = _sample(T)
    ref = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  inp.ws_gate, inp.ws_up, inp.ws_down, M=cfg.M, kp=cfg.kp, dtype=cfg.dtype,
                  logits_f32=scores, tokens=tok)
    err = normwise_rel_err(values(out["y"])[tok], ref["y"])
    assert err <= tolerance(cfg), err


def _score_error_bound(inp, cfg):
    """Bound on |float32 scores - exact scores| for any summation order:
    (d + 2) * 2^-24 * sum_j |x_j w_j|, plus one rounding of the bias add,
    2^-24 * (sum_j |x_j w_j| + |b|) (the computed score is at most that in size)."""
    x = O.to_f64(inp.x, cfg.dtype)
    w = O.to_f64(inp.w_router, cfg.dtype)
    s = np.abs(x) @ np.abs(w).T
    b = 0.0 if inp.router_bias is None else np.abs(np.asarray(inp.router_bias, np.float64))[None, :]
    return (cfg.d + 2) * 2.0 ** -24 * s + 2.0 ** -24 * (s + b) + 1e-30


@pytest.mark.parametrize("name,T", [("C0", 64), ("C1", 64), ("C2", 456), ("C3", 4096),
                                    ("C4", 16384)])
def test_layer_full(lib, name, T):
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    say("layer (full)", name, T)
    out = _run_layer(lib, cfg, T, dw)
    tok = _sample(T)
    ref = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  inp.ws_gate, inp.ws_up, inp.ws_down, M=cfg.M, kp=cfg.kp, dtype=cfg.dtype,
                  tokens=tok)
    # scores within the float32 summation bound of the exact ones
    bound = _score_error_bound(inp, cfg)
    assert (np.abs(out["logits"] - ref["logits64"]) <= bound).all()
    # routing: identical except where two experts' exact scores are within the bound
    diff = np.nonzero((out["idx"] != ref["idx"]).any(1))[0]
    for t in diff:
        for k in np.nonzero(out["idx"][t] != ref["idx"][t])[0]:
            a, b = out["idx"][t, k], ref["idx"][t, k]
            assert abs(ref["logits64"][t, a] - ref["logits64"][t, b]) <= bound[t, a] + bound[t, b]
    assert len(diff) <= max(2, T // 1000)
    assert (out["gc"] == T * cfg.kp).all()
    same = np.array([t not in set(diff.tolist()) for t in tok])
    err = normwise_rel_err(values(out["y"])[tok][same], ref["y"][same])
    assert err <= tolerance(cfg), err


# ----------------------------------------------------------------------------
# the routed experts alone at full size
# ----------------------------------------------------------------------------
# In the layer output the ungated shared experts dominate (the routed part is
# under a tenth of max|y| at the decode batch), so a normwise bound on y says
# little about the routed experts.  These run the layer with no shared experts
# (shared_inter = 0, the same routed weights), so y is the gate-weighted sum of the
# routed experts alone; the layer reads each row of x through sorted_pair inside
# the 64-row (T=456) and 256-row (T=4096, 16384) tile kernels at d = 5120.

def _routed_dims(lib, cfg, T):
    return lib.make_dims(T, cfg.d, cfg.N, cfg.M, cfg.kp, cfg.inter, 0,
                         lib.MOGE_BF16 if cfg.dtype == "bf16" else lib.MOGE_F32)


def _run_routed_layer(lib, cfg, T, dw, scores, packed=None):
    import torch
    dims = _routed_dims(lib, cfg, T)
    y = _empty((T, cfg.d), dw["x"].dtype)
    idx = _empty((T, dims.K), torch.int32)
    gc = _empty((cfg.M,), torch.int32)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    if packed is None:
        lib.layer_forward(dims, dw["x"], None, None, dw["w_gate"], dw["w_up"], dw["w_down"],
                          None, None, None, y, ws, logits_in=to_dev(scores, "f32"),
                          topk_idx_out=idx, group_counts_out=gc)
    else:
        lib.layer_forward_packed(dims, dw["x"], None, None, packed, y, ws,
                                 logits_in=to_dev(scores, "f32"), topk_idx_out=idx,
                                 group_counts_out=gc)
    torch.cuda.synchronize()
    return to_host(y), to_host(idx), to_host(gc)


def _no_shared(cfg):
    z = np.zeros((0, cfg.d), dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    return z, z, np.ascontiguousarray(z.T)


def elementwise_rel_err(y, ref, floor_frac=1e-2):
    """Elementwise |y - ref| / |ref| over the elements with |ref| at least
    floor_frac * max|ref| (a diagnostic beside the normwise measure): max and
    99.9th percentile."""
    den = np.abs(ref)
    m = den >= floor_frac * den.max()
    r = np.abs(y - ref)[m] / den[m]
    return float(r.max()), float(np.quantile(r, 0.999))


# (12000 tokens: just enough 256-row gate/up tiles for persistent workgroups in
# rounds, with a partial last round and list entries that name no tile)
@pytest.mark.parametrize("name,T,n_tok", [("C2", 456, None), ("C3", 4096, 256),
                                          ("C4", 12000, 256), ("C4", 16384, 256)])
def test_layer_routed_only_full_size(lib, name, T, n_tok):
    import torch
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    say("layer routed only (row-major)", name, T)
    y, idx, gc = _run_routed_layer(lib, cfg, T, dw, scores)
    r = O.route(scores, cfg.M, cfg.kp)
    np.testing.assert_array_equal(idx, r["idx"])
    assert (gc == T * cfg.kp).all()
    # the packed layer gives the same bits
    dims = _routed_dims(lib, cfg, T)
    packed = _empty(lib.packed_weights_size(dims), torch.uint8)
    lib.pack_weights(dims, dw["w_gate"], dw["w_up"], dw["w_down"], None, None, None, packed)
    say("layer routed only (packed)", name, T)
    yp, idxp, _ = _run_routed_layer(lib, cfg, T, dw, scores, packed=packed)
    del packed
    np.testing.assert_array_equal(idxp, idx)
    np.testing.assert_array_equal(yp, y)
    tok = np.arange(T) if n_tok is None else S.sample_tokens(T, n_tok)
    zg, zu, zd = _no_shared(cfg)
    ref = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  zg, zu, zd, M=cfg.M, kp=cfg.kp, dtype=cfg.dtype, logits_f32=scores, tokens=tok)
    got = values(y)[tok]
    err = normwise_rel_err(got, ref["y"])
    emax, e999 = elementwise_rel_err(got, ref["y"])
    print(f"[routed-only {name}] tokens {len(tok)}: normwise {err:.3e}, elementwise "
          f"(|ref| >= 1e-2 max) max {emax:.3e}, p99.9 {e999:.3e}", flush=True)
    assert err <= tolerance(cfg), err
    assert np.isfinite(values(y)).all()


@pytest.mark.parametrize("name,T", [("C2", 456), ("C3", 4096), ("C4", 12000), ("C4", 16384)])
def test_layer_routed_only_equals_step_path_bitwise(lib, name, T):
    # the layer's gather through sorted_pair against the step path's materialised
    # x_perm, with no shared experts: the same kernels on the same rows, bit for bit
    # (the step path runs one 256-row tile per workgroup, the layer at 12000 and
    # 16384 tokens persistent workgroups in rounds: the order of tiles does not
    # change a result)
    import torch
    cfg = CONFIGS[name]
    _, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    say("layer routed only vs step path", name, T)
    y_layer, _, _ = _run_routed_layer(lib, cfg, T, dw, scores)
    dims = _routed_dims(lib, cfg, T)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    idx = _empty((T, dims.K), torch.int32)
    gate = _empty((T, dims.K), torch.float32)
    lib.route(dims, to_dev(scores, "f32"), idx, gate)
    i32 = lambda n: _empty(n, torch.int32)
    counts, offsets, gc, sp, pr = i32(cfg.N), i32(cfg.N + 1), i32(cfg.M), i32(dims.R), i32(dims.R)
    x_perm = _empty((dims.R, cfg.d), dw["x"].dtype)
    lib.permute(dims, idx, dw["x"], counts, offsets, gc, sp, pr, x_perm, ws)
    y_perm = _empty((dims.R, cfg.d), dw["x"].dtype)
    lib.expert_ffn(dims, x_perm, offsets, dw["w_gate"], dw["w_up"], dw["w_down"], y_perm, ws)
    del x_perm
    y = _empty((T, cfg.d), dw["x"].dtype)
    lib.combine(dims, y_perm, pr, gate, None, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(y), y_layer)


def test_layer_zero_tokens(lib):
    import torch
    cfg = C1
    dims = dims_of(lib, cfg, 0)
    _, dw = layer_inputs(cfg, 1)
    y = torch.full((1, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = _empty(max(256, lib.workspace_size(dims)), torch.uint8)
    say("layer T=0")
    lib.layer_forward(dims, dw["x"], dw["w_router"], None, dw["w_gate"], dw["w_up"], dw["w_down"],
                      dw["ws_gate"], dw["ws_up"], dw["ws_down"], y, ws)
    torch.cuda.synchronize()
    assert (y.float() == 7.0).all()


@pytest.mark.parametrize("name,T", [("C1", 64), ("C1", 456), ("C0", 200)])
def test_layer_one_expert_per_group_takes_everything(lib, name, T):
    # the first expert of every group wins every token: each active expert gets
    # all T rows, the others none (degenerate but balanced routing)
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    scores[:, ::cfg.G] += 50.0
    say("layer one-expert-per-group", name, T)
    out = _run_layer(lib, cfg, T, dw, logits_in=scores)
    np.testing.assert_array_equal(out["idx"], O.route(scores, cfg.M, cfg.kp)["idx"])
    tok = _sample(T)
    ref = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  inp.ws_gate, inp.ws_up, inp.ws_down, M=cfg.M, kp=cfg.kp, dtype=cfg.dtype,
                  logits_f32=scores, tokens=tok)
    assert normwise_rel_err(values(out["y"])[tok], ref["y"]) <= tolerance(cfg)


# split_shared: the layer splits the shared experts' contraction (a 64-token batch:
# both projections; 456 tokens: the down projection, whose shared tiles run beside
# the routed ones); elsewhere the layer equals the step path bit for bit
@pytest.mark.parametrize("name,T,split_shared", [("C0", 64, False), ("C1", 64, True),
                                                 ("C1", 17, False), ("C2", 456, True)])
def test_layer_deterministic_and_equal_to_step_path(lib, name, T, split_shared):
    import torch
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    say("determinism + step path", name, T)
    a = _run_layer(lib, cfg, T, dw, logits_in=scores)
    b = _run_layer(lib, cfg, T, dw, logits_in=scores)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    f = _run_layer(lib, cfg, T, dw)
    g = _run_layer(lib, cfg, T, dw)
    for k in f:
        np.testing.assert_array_equal(f[k], g[k], err_msg=k)
    # the same layer through the five step entry points
    dims = dims_of(lib, cfg, T)
    ws = _empty(lib.workspace_size(dims), torch.uint8)
    idx = _empty((T, dims.K), torch.int32)
    gate = _empty((T, dims.K), torch.float32)
    lib.route(dims, to_dev(scores, "f32"), idx, gate)
    i32 = lambda n: _empty(n, torch.int32)
    counts, offsets, gc, sp, pr = i32(cfg.N), i32(cfg.N + 1), i32(cfg.M), i32(dims.R), i32(dims.R)
    x_perm = _empty((dims.R, cfg.d), dw["x"].dtype)
    lib.permute(dims, idx, dw["x"], counts, offsets, gc, sp, pr, x_perm, ws)
    y_perm = _empty((dims.R, cfg.d), dw["x"].dtype)
    lib.expert_ffn(dims, x_perm, offsets, dw["w_gate"], dw["w_up"], dw["w_down"], y_perm, ws)
    sdims = lib.make_dims(T, cfg.d, 1, 1, 1, cfg.I_s, 0, dims.dtype)
    sws = _empty(lib.workspace_size(sdims), torch.uint8)
    sh = _empty((T, cfg.d), dw["x"].dtype)
    lib.expert_ffn(sdims, dw["x"], to_dev(np.array([0, T], dtype=np.int32), "f32"),
                   dw["ws_gate"], dw["ws_up"], dw["ws_down"], sh, sws)
    y = _empty((T, cfg.d), dw["x"].dtype)
    lib.combine(dims, y_perm, pr, gate, sh, y)
    torch.cuda.synchronize()
    if split_shared:
        # the layer splits the shared experts' contraction over several tiles and
        # adds the float32 partial sums without the step path's bf16 rounding of the
        # shared output (and of H_s, where gate/up is split too): the results
        # differ by those roundings
        err = normwise_rel_err(values(to_host(y)), values(a["y"]))
        assert 0 < err <= 2 * 2.0 ** -8, err
    else:
        np.testing.assert_array_equal(to_host(y), a["y"])
