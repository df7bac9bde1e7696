"""Pins for the CPU oracle: checks against closed forms, brute force, textbook
routines other than the ones the oracle calls, and the invariants the pages fix
(TechWalker "Huawei releases Pangu Pro MoE" sections 一 and 六; Reportify concept
page "分组混合专家模型", 技术创新细节).  None of these tests re-types the oracle's own
formula: each one computes the expected value another way."""
import heapq
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import moge_oracle as O
from synth import inputs as S
from synth.configs import C0, C1, C4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------
# S1 softmax
# ----------------------------------------------------------------------------

def test_softmax_closed_form():
    # scores ln(1), ln(2), ln(3): probabilities 1/6, 2/6, 3/6 exactly
    l = np.log(np.array([[1.0, 2.0, 3.0]]))
    np.testing.assert_allclose(O.softmax(l), [[1 / 6, 2 / 6, 3 / 6]], rtol=0, atol=1e-15)


def test_softmax_matches_scipy_and_sums_to_one():
    l = _rng(1).normal(size=(50, 64)) * 4
    p = O.softmax(l)
    np.testing.assert_allclose(p, scipy.special.softmax(l, axis=1), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
    assert (p > 0).all()


def test_softmax_shift_invariant_and_large_scores():
    l = _rng(2).normal(size=(8, 16))
    np.testing.assert_allclose(O.softmax(l + 1000.0), O.softmax(l), rtol=1e-12)
    # all-equal scores: uniform
    np.testing.assert_allclose(O.softmax(np.zeros((3, 8))), 1 / 8, atol=1e-16)


def test_softmax_rejects_nonfinite():
    with pytest.raises(ValueError):
        O.softmax(np.array([[0.0, np.nan]]))


# ----------------------------------------------------------------------------
# S2 grouped top-K'
# ----------------------------------------------------------------------------

def _brute_force_select(row, M, kp):
    """Enumerate every expert subset with exactly kp experts from each of the M
    contiguous groups; keep the one with the largest score sum; on equal sums
    the lexicographically smallest sorted index tuple.  Integer scores keep the
    sums exact."""
    N = len(row)
    G = N // M
    per_group = [list(itertools.combinations(range(g * G, (g + 1) * G), kp)) for g in range(M)]
    best, best_key = None, None
    for choice in itertools.product(*per_group):
        sel = tuple(sorted(itertools.chain(*choice)))
        total = sum(int(row[e]) for e in sel)
        key = (-total, sel)
        if best_key is None or key < best_key:
            best, best_key = sel, key
    return best


@pytest.mark.parametrize("N,M,kp", [(4, 1, 2), (6, 2, 1), (6, 3, 1), (8, 2, 2), (8, 4, 1),
                                    (9, 3, 2), (12, 4, 2), (12, 3, 3), (8, 1, 3), (6, 2, 3)])
def test_group_topk_brute_force(N, M, kp):
    rng = _rng(N * 100 + M * 10 + kp)
    scores = rng.integers(-2, 3, size=(40, N)).astype(np.float32)   # many ties
    idx = O.group_topk(scores, M, kp)
    G = N // M
    for t in range(scores.shape[0]):
        assert tuple(sorted(idx[t].tolist())) == _brute_force_select(scores[t], M, kp)
        # slot order inside a group: score descending, index ascending on ties
        for g in range(M):
            slots = idx[t, g * kp:(g + 1) * kp].tolist()
            keys = [(-scores[t, e], e) for e in slots]
            assert keys == sorted(keys)
            assert all(g * G <= e < (g + 1) * G for e in slots)


def test_global_topk_matches_heapq():
    rng = _rng(3)
    scores = rng.integers(-3, 4, size=(60, 16)).astype(np.float32)
    for K in (1, 3, 8, 16):
        got = O.global_topk(scores, K)
        for t in range(scores.shape[0]):
            ref = heapq.nlargest(K, range(16), key=lambda e: (scores[t, e], -e))
            assert got[t].tolist() == ref


def test_exactly_kp_per_group_and_distinct():
    rng = _rng(4)
    for (N, M, kp) in [(64, 8, 1), (64, 8, 2), (256, 8, 4), (16, 4, 1), (64, 64, 1)]:
        s = rng.normal(size=(100, N)).astype(np.float32)
        idx = O.group_topk(s, M, kp)
        G = N // M
        assert idx.shape == (100, M * kp)
        grp = idx // G
        for g in range(M):
            assert (np.sum(grp == g, axis=1) == kp).all()
        assert all(len(set(r)) == M * kp for r in idx.tolist())


def test_kp_equal_G_selects_every_expert():
    s = _rng(5).normal(size=(20, 12)).astype(np.float32)
    idx = O.group_topk(s, 3, 4)
    assert (np.sort(idx, axis=1) == np.arange(12)).all()


def test_no_coactivation_inside_a_group_when_kp_is_1():
    # expert analysis section: with one expert per group, two experts of one group
    # are never active for the same token
    s = _rng(6).normal(size=(500, 64)).astype(np.float32)
    idx = O.group_topk(s, 8, 1)
    co = np.zeros((64, 64), dtype=np.int64)
    for row in idx:
        for a in row:
            for b in row:
                if a != b:
                    co[a, b] += 1
    for g in range(8):
        assert co[g * 8:(g + 1) * 8, g * 8:(g + 1) * 8].sum() == 0
    assert co.sum() > 0


def test_routing_golden_example():
    with open(os.path.join(GOLDEN, "routing_small.json")) as f:
        gd = json.load(f)
    w0 = np.array(gd["weights_row0"], dtype=np.float64)
    row0 = np.log(w0).astype(np.float32)
    row1 = np.array([float(v) for v in gd["scores_row1"]], dtype=np.float32)
    assert math.copysign(1, row1[1]) < 0 and math.copysign(1, row1[0]) > 0
    scores = np.stack([row0, row1])
    ex = gd["expected"]
    for kp, key in ((1, "kp1"), (2, "kp2")):
        r = O.route(scores, gd["M"], kp)
        assert r["idx"][0].tolist() == ex[key]["idx_row0"]
        assert r["idx"][1].tolist() == ex[key]["idx_row1"]
        want = [eval(fr) for fr in ex[key]["gate_row0"]]   # fractions like "3/18"
        np.testing.assert_allclose(r["gate"][0], want, rtol=1e-6)
    r1 = O.route(scores, 2, 1)
    z = 5 + math.exp(-1) + math.exp(-2) + math.exp(-3)
    np.testing.assert_allclose(r1["gate"][1], [1 / z, 1 / z], rtol=1e-12)
    assert O.global_topk(scores, 3)[0].tolist() == ex["global_top3_row0"]


def test_router_scores_golden_example():
    # S0 with a per-expert bias: hand-worked integer scores, and a bias that flips
    # one group's choice for each token (tests/golden/router_scores_small.json)
    with open(os.path.join(GOLDEN, "router_scores_small.json")) as f:
        gd = json.load(f)
    ex = gd["expected"]
    x = np.array(gd["x"], dtype=np.float32)
    w = np.array(gd["w_router"], dtype=np.float32)
    b = np.array(gd["bias"], dtype=np.float32)
    M, kp = gd["M"], gd["kp"]
    # scores, exactly (small integers)
    assert O.router_logits(x.astype(np.float64), w.astype(np.float64)).tolist() == \
        ex["scores_no_bias"]
    assert O.router_logits(x.astype(np.float64), w.astype(np.float64), b).tolist() == \
        ex["scores_with_bias"]
    # the same scores by an element loop over the stored integers
    for t in range(2):
        for e in range(8):
            v = sum(gd["x"][t][j] * gd["w_router"][e][j] for j in range(3))
            assert ex["scores_no_bias"][t][e] == v
            assert ex["scores_with_bias"][t][e] == v + gd["bias"][e]
    # through the whole layer: the bias goes in before the softmax and the selection
    N, d, I = 8, 3, 2
    z = np.zeros
    for bias, key in ((None, "no_bias"), (b, "with_bias")):
        out = O.layer(x, w, bias, z((N, I, d), np.float32), z((N, I, d), np.float32),
                      z((N, d, I), np.float32), z((2, d), np.float32), z((2, d), np.float32),
                      z((d, 2), np.float32), M=M, kp=kp, dtype="f32")
        assert out["logits64"].tolist() == ex["scores_" + key]
        assert out["idx"].tolist() == ex["idx_" + key]
        assert (out["y"] == 0).all()
    e = math.e
    g0 = e ** 2 / (3 * e + 2 * e ** 2 + e ** -3 + 1 + e ** -1)
    g1 = e ** 6 / (2 + 2 * e ** 4 + e ** 6 + e ** 3 + e ** -1 + e ** -4)
    np.testing.assert_allclose(out["gate"][0], [g0, g0], rtol=1e-6)
    np.testing.assert_allclose(out["gate"][1], [g1, g1 / e ** 2], rtol=1e-6)


def test_gate_is_unnormalised_global_probability():
    # the gate is the probability from the softmax over all N experts, so the K
    # gates of a token sum to less than 1 when K < N
    s = _rng(7).normal(size=(30, 16)).astype(np.float32)
    r = O.route(s, 4, 1)
    e = np.exp(s.astype(np.float64))
    for t in range(30):
        for k in range(4):
            assert abs(r["gate"][t, k] - e[t, r["idx"][t, k]] / e[t].sum()) < 1e-15
    assert (r["gate"].sum(1) < 1).all()


# ----------------------------------------------------------------------------
# S3 permutation, group loads, imbalance score
# ----------------------------------------------------------------------------

def test_permute_matches_python_sort():
    rng = _rng(8)
    s = rng.normal(size=(37, 16)).astype(np.float32)
    idx = O.group_topk(s, 4, 2)
    T, K = idx.shape
    p = O.permute(idx, 16, 4)
    pairs = sorted(range(T * K), key=lambda q: (idx[q // K, q % K], q // K))
    assert p["sorted_pair"].tolist() == pairs
    assert (p["sorted_pair"][p["pair_row"]] == np.arange(T * K)).all()
    assert p["counts"].tolist() == [int(np.sum(idx == e)) for e in range(16)]
    assert p["offsets"][0] == 0 and p["offsets"][-1] == T * K
    assert (np.diff(p["offsets"]) == p["counts"]).all()


def test_group_loads_equal_imbalance_zero():
    for cfg in (C0, C1, C4):
        s = S.make_scores(cfg, T=min(cfg.T, 2048))
        T = s.shape[0]
        idx = O.group_topk(s, cfg.M, cfg.kp)
        p = O.permute(idx, cfg.N, cfg.M)
        assert (p["group_counts"] == T * cfg.kp).all()
        assert O.imbalance_score(p["group_counts"], T) == 0.0


def test_global_topk_is_imbalanced_under_zipf_bias():
    s = S.make_scores(C4, T=2048)
    g = O.global_topk(s, 8)
    loads = O.group_loads_of(g, 64, 8)
    assert loads.sum() == 2048 * 8
    # favoured low-numbered experts sit in the first groups
    assert loads[0] > loads[-1]
    assert O.imbalance_score(loads, 2048) > 1.0
    # the hand-computable extreme: identical scores for every token make global
    # top-K take experts 0..K-1, i.e. all of group 0 when K = G
    flat = np.tile(np.arange(64, 0, -1, dtype=np.float32), (10, 1))
    assert O.imbalance_score(O.group_loads_of(O.global_topk(flat, 8), 64, 8), 10) == 8.0


def test_imbalance_score_closed_form():
    assert O.imbalance_score([5, 5, 5], 5) == 0.0
    assert O.imbalance_score([9, 1, 5], 4) == 2.0


def test_expert_share_near_one_over_G():
    # with independent scores every expert of a group of 8 gets about 12.5 % of its
    # group's tokens (expert analysis section); a chi-square sanity check
    T = 16000
    s = S.normal_tensor((T, 64), 1.0, 11, 8, "f32")
    idx = O.group_topk(s, 8, 1)
    c = np.bincount(idx.reshape(-1), minlength=64).reshape(8, 8)
    from scipy.stats import chisquare
    for g in range(8):
        assert chisquare(c[g]).pvalue > 1e-4
        np.testing.assert_allclose(c[g] / T, 0.125, atol=0.015)


# ----------------------------------------------------------------------------
# S4-S6 SwiGLU FFN: closed forms
# ----------------------------------------------------------------------------

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    np.testing.assert_allclose(O.silu(np.array([0.0, ln3, -ln3])), [0.0, 0.75 * ln3, -0.25 * ln3],
                               rtol=1e-15, atol=0)
    np.testing.assert_allclose(O.silu(np.array([40.0])), [40.0], rtol=1e-15)
    np.testing.assert_allclose(O.silu(np.array([-50.0])), [0.0], atol=1e-18)


def test_swiglu_closed_form_scalar():
    ln3 = math.log(3.0)
    # x = 2, wg = ln3/2 -> gate ln3; wu = 1.5 -> up 3; wd = 0.5
    y = O.swiglu(np.array([[2.0]]), np.array([[ln3 / 2]]), np.array([[1.5]]), np.array([[0.5]]))
    assert abs(y[0, 0] - 1.125 * ln3) < 1e-15


def test_swiglu_closed_form_asymmetric():
    # operands chosen so that a transposed weight anywhere changes the result
    ln3 = math.log(3.0)
    X = np.array([[1.0, 2.0]])
    Wg = np.array([[0.0, ln3 / 2], [0.0, 0.0]])      # gate = (ln3, 0)
    Wu = np.array([[1.0, 1.0], [2.0, 0.0]])           # up   = (3, 2)
    Wd = np.array([[1.0, 5.0], [-2.0, 7.0]])          # h = (2.25 ln3, 0)
    y = O.swiglu(X, Wg, Wu, Wd)
    np.testing.assert_allclose(y, [[2.25 * ln3, -4.5 * ln3]], rtol=1e-15)


def _brute_ffn(xrow, Wg, Wu, Wd):
    """Element-by-element SwiGLU for one token (loops, no matmul)."""
    I, d = Wg.shape
    h = []
    for i in range(I):
        a = sum(xrow[j] * Wg[i, j] for j in range(d))
        b = sum(xrow[j] * Wu[i, j] for j in range(d))
        h.append(a / (1.0 + math.exp(-a)) * b)
    return np.array([sum(h[i] * Wd[o, i] for i in range(I)) for o in range(Wd.shape[0])])


def _tiny_inputs(N=8, M=2, d=6, I=4, Is=6, T=9, seed=0, dtype="f32"):
    rng = _rng(seed)
    def a(*shape, sd=0.5):
        return (rng.normal(size=shape) * sd).astype(np.float32)
    return dict(x=a(T, d, sd=1.0), w_router=a(N, d), router_bias=None,
                w_gate=a(N, I, d), w_up=a(N, I, d), w_down=a(N, d, I),
                ws_gate=a(Is, d), ws_up=a(Is, d), ws_down=a(d, Is))


@pytest.mark.parametrize("kp", [1, 2])
def test_layer_equals_dense_brute_force(kp):
    # the permuted/combined layer equals the per-token dense definition written
    # with loops: y_t = shared(x_t) + sum over chosen experts of p * FFN_e(x_t)
    N, M = 8, 2
    inp = _tiny_inputs(N=N, M=M, seed=kp)
    out = O.layer(**inp, M=M, kp=kp, dtype="f32")
    x = inp["x"].astype(np.float64)
    l = x @ inp["w_router"].astype(np.float64).T
    l32 = l.astype(np.float32)
    e = np.exp(l32.astype(np.float64))
    p = e / e.sum(1, keepdims=True)
    G = N // M
    for t in range(x.shape[0]):
        y = _brute_ffn(x[t], inp["ws_gate"].astype(np.float64), inp["ws_up"].astype(np.float64),
                       inp["ws_down"].astype(np.float64))
        for g in range(M):
            grp = sorted(range(g * G, (g + 1) * G), key=lambda q: (-l32[t, q], q))[:kp]
            for q in grp:
                y = y + p[t, q] * _brute_ffn(x[t], inp["w_gate"][q].astype(np.float64),
                                             inp["w_up"][q].astype(np.float64),
                                             inp["w_down"][q].astype(np.float64))
        np.testing.assert_allclose(out["y"][t], y, rtol=1e-12, atol=1e-14)


def test_shared_experts_concatenation_identity():
    # S separate SwiGLU experts summed == one SwiGLU of width S*I with the weights
    # concatenated along the intermediate dimension
    rng = _rng(9)
    d, I, Sn = 5, 3, 4
    f32 = lambda *shape: rng.normal(size=shape).astype(np.float32).astype(np.float64)
    x = f32(7, d)
    parts = [(f32(I, d), f32(I, d), f32(d, I)) for _ in range(Sn)]
    want = np.zeros((7, d))
    for t in range(7):
        for (g, u, dn) in parts:
            want[t] += _brute_ffn(x[t], g, u, dn)
    got = O.shared_experts(x, np.concatenate([p[0] for p in parts]),
                           np.concatenate([p[1] for p in parts]),
                           np.concatenate([p[2] for p in parts], axis=1), "f32")
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_kp_equal_G_gives_dense_mixture():
    N, M = 6, 2
    inp = _tiny_inputs(N=N, M=M, seed=5)
    out = O.layer(**inp, M=M, kp=N // M, dtype="f32")
    x = inp["x"].astype(np.float64)
    l32 = (x @ inp["w_router"].astype(np.float64).T).astype(np.float32)
    p = scipy.special.softmax(l32.astype(np.float64), axis=1)
    for t in range(x.shape[0]):
        y = _brute_ffn(x[t], inp["ws_gate"].astype(np.float64), inp["ws_up"].astype(np.float64),
                       inp["ws_down"].astype(np.float64))
        for q in range(N):
            y = y + p[t, q] * _brute_ffn(x[t], inp["w_gate"][q].astype(np.float64),
                                         inp["w_up"][q].astype(np.float64),
                                         inp["w_down"][q].astype(np.float64))
        np.testing.assert_allclose(out["y"][t], y, rtol=1e-12, atol=1e-14)


def test_zero_routed_down_weights_leave_shared_only():
    inp = _tiny_inputs(seed=6)
    inp["w_down"] = np.zeros_like(inp["w_down"])
    out = O.layer(**inp, M=2, kp=1, dtype="f32")
    np.testing.assert_array_equal(out["y"], out["shared"])


def test_combine_closed_form():
    # two tokens, K=2, three permuted rows; hand-computed sums
    y_perm = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0], [5.0, 5.0]])
    pair_row = np.array([2, 0, 1, 3])          # token0 -> rows 2,0; token1 -> rows 1,3
    gate = np.array([[0.5, 0.25], [0.1, 1.0]])
    sh = np.array([[1.0, 1.0], [0.0, -1.0]])
    y = O.combine(y_perm, pair_row, gate, sh, 2, 2)
    np.testing.assert_allclose(y, [[1 + 50 + 0.25, 1 + 100 + 0.5], [1 + 5, -1 + 2 + 5]], rtol=1e-15)


def test_bf16_widening_exact():
    # bf16 0x3F80 = 1.0, 0xC000 = -2.0, 0x3EAB = 0.333984375, 0x0001 = 2^-133
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0001], dtype=np.uint16)
    np.testing.assert_array_equal(O.to_f64(bits, "bf16"), [1.0, -2.0, 0.333984375, 2.0 ** -133])


def test_layer_token_subset_matches_full():
    inp = _tiny_inputs(seed=7, T=12)
    full = O.layer(**inp, M=2, kp=1, dtype="f32")
    sub = O.layer(**inp, M=2, kp=1, dtype="f32", tokens=np.array([0, 5, 11]))
    np.testing.assert_allclose(sub["y"], full["y"][[0, 5, 11]], rtol=1e-13, atol=1e-15)


def test_c0_layer_runs_fast_and_is_balanced():
    inp = S.make_layer_inputs(C0)
    out = O.layer(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                  inp.ws_gate, inp.ws_up, inp.ws_down, M=C0.M, kp=C0.kp, dtype="f32")
    assert out["y"].shape == (C0.T, C0.d)
    assert (out["group_counts"] == C0.T).all()
    assert np.isfinite(out["y"]).all()


# ----------------------------------------------------------------------------
# int8 expert weights (reading Q1)
# ----------------------------------------------------------------------------

def test_w8_quantize_golden_rows():
    with open(os.path.join(GOLDEN, "w8_quantize_small.json")) as f:
        g = json.load(f)
    q, s = O.w8_quantize(np.array(g["rows"], dtype=np.float32), "f32")
    np.testing.assert_array_equal(s, np.array(g["scales"], dtype=np.float32))
    np.testing.assert_array_equal(q, np.array(g["codes"], dtype=np.int8))
    assert q.dtype == np.int8 and s.dtype == np.float32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_w8_quantize_error_bound_and_range(dtype):
    # every code is within half a step of the weight it stands for, the largest
    # weight of a row maps to +-127, and no code leaves [-127, 127]
    rng = _rng(31)
    w = (rng.standard_t(3, size=(40, 3, 96)) * 0.02).astype(np.float32)
    w[3, 1] = 0.0
    wb = S.f32_to_bf16_bits(w) if dtype == "bf16" else w
    q, s = O.w8_quantize(wb, dtype)
    w64 = S.bf16_bits_to_f32(wb).astype(np.float64) if dtype == "bf16" else w.astype(np.float64)
    s64 = s.astype(np.float64)[..., None]
    assert q.shape == w.shape and s.shape == w.shape[:-1]
    assert np.abs(q.astype(np.int64)).max() <= 127
    assert (np.abs(q.astype(np.float64) * s64 - w64) <= s64 * (0.5 + 1e-5)).all()
    nz = np.abs(w64).max(-1) > 0
    assert (np.abs(q.astype(np.int64)).max(-1)[nz] == 127).all()
    assert (s[~nz] == 0).all() and (q[~nz] == 0).all()


def _exact_w8_weights(rng, *shape):
    """float32 weights whose rows are integers (largest magnitude 127) times a
    power of two, with the codes and scales they quantise to by construction."""
    ints = rng.integers(-127, 128, size=shape)
    flat = ints.reshape(-1, shape[-1])
    for r in range(flat.shape[0]):
        flat[r, rng.integers(shape[-1])] = 127 if rng.random() < 0.5 else -127
    ints = flat.reshape(shape)
    e = rng.integers(6, 10, size=shape[:-1]).astype(np.float64)
    scale = np.exp2(-e)
    w = (ints * scale[..., None]).astype(np.float32)
    return w, ints.astype(np.int8), scale.astype(np.float32)


def test_w8_layer_is_the_layer_on_exactly_quantisable_weights():
    # weights that are exactly integers times a per-row power of two quantise to
    # those integers and scales, and the int8 layer on them is the float layer
    rng = _rng(33)
    N, M, d, I, Is, T = 6, 2, 8, 4, 6, 9
    wg, qg, sg = _exact_w8_weights(rng, N, I, d)
    wu, qu, su = _exact_w8_weights(rng, N, I, d)
    wd, qd, sd = _exact_w8_weights(rng, N, d, I)
    wsg, qsg, ssg = _exact_w8_weights(rng, Is, d)
    wsu, qsu, ssu = _exact_w8_weights(rng, Is, d)
    wsd, qsd, ssd = _exact_w8_weights(rng, d, Is)
    for w, q, s in ((wg, qg, sg), (wd, qd, sd), (wsd, qsd, ssd)):
        q2, s2 = O.w8_quantize(w, "f32")
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, s)
    x = rng.normal(size=(T, d)).astype(np.float32)
    wr = rng.normal(size=(N, d)).astype(np.float32)
    ref = O.layer(x, wr, None, wg, wu, wd, wsg, wsu, wsd, M=M, kp=1, dtype="f32")
    got = O.layer_w8(x, wr, None, qg, sg, qu, su, qd, sd, qsg, ssg, qsu, ssu, qsd, ssd, M=M,
                     kp=1, dtype="f32")
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["y"], ref["y"])
