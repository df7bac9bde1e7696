"""Weight-only int8 experts on the GPU, through the C ABI, against the oracle.

* moge_pack_weights_w8 writes exactly the layout include/moge.h defines (bytes).
* moge_quantize_weights_w8 gives the oracle's codes and scales bit for bit (every
  decision in float32 on both sides).
* moge_layer_forward_w8 routes exactly like the oracle and its output is within
  the bf16 layer tolerance of the oracle's layer on the weights s * q, at small
  ragged sizes that reach every row-subtile count (1..4 subtiles of 16 rows, and
  several 64-row passes) and at the decode workloads' full sizes (sampled tokens).
"""
import functools
from dataclasses import replace

import numpy as np
import pytest

from oracle import moge_oracle as O
from synth import inputs as S
from synth.configs import C0, C1, C2, C3
from tests import packed_ref
from tests.gpu_util import (dims_of, layer_inputs, normwise_rel_err, say, to_dev, to_host,
                            tolerance, values, weight_key)

# small int8 layers: d = 256, I = 128, I_s = 256 with one expert per group (K = 4),
# and I = 192, I_s = 384 with two experts per group (K = 8)
W1 = replace(C0, name="W8-small", dtype="bf16")
W2 = replace(C0, name="W8-small-kp2", dtype="bf16", kp=2, inter=192, shared_inter=384)
CONFIGS = {"W1": W1, "W2": W2, "C1": C1, "C2": C2, "C3": C3}


def _empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


@functools.lru_cache(maxsize=1)
def _w8_host(key):
    return S.make_w8_weights(key)


@functools.lru_cache(maxsize=1)
def _w8_dev(key):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in _w8_host(key).items()}


def _w8_buffer(lib, cfg, dims):
    w = _w8_dev(weight_key(cfg))
    buf = _empty((lib.w8_weights_size(dims),), __import__("torch").uint8)
    lib.pack_weights_w8(dims, w["q_gate"], w["q_up"], w["q_down"], w["s_gate"], w["s_up"],
                        w["s_down"], w["qs_gate"], w["qs_up"], w["qs_down"], w["ss_gate"],
                        w["ss_up"], w["ss_down"], buf)
    return buf


def _run(lib, cfg, T, dw, buf, logits_in=None):
    import torch
    dims = dims_of(lib, cfg, T)
    out = dict(y=_empty((T, cfg.d), torch.bfloat16), logits=_empty((T, cfg.N), torch.float32),
               idx=_empty((T, dims.K), torch.int32), gate=_empty((T, dims.K), torch.float32),
               gc=_empty((cfg.M,), torch.int32))
    ws = _empty((lib.workspace_size(dims),), torch.uint8)
    lib.layer_forward_w8(dims, dw["x"], dw["w_router"], dw["router_bias"], buf, out["y"], ws,
                         logits_in=None if logits_in is None else to_dev(logits_in, "f32"),
                         logits_out=out["logits"], topk_idx_out=out["idx"],
                         topk_gate_out=out["gate"], group_counts_out=out["gc"])
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _oracle(inp, w, cfg, scores, tok):
    return O.layer_w8(inp.x, inp.w_router, inp.router_bias, w["q_gate"], w["s_gate"],
                      w["q_up"], w["s_up"], w["q_down"], w["s_down"], w["qs_gate"], w["ss_gate"],
                      w["qs_up"], w["ss_up"], w["qs_down"], w["ss_down"], M=cfg.M, kp=cfg.kp,
                      dtype=cfg.dtype, logits_f32=scores, tokens=tok)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["W1", "W2", "C1"])
def test_w8_pack_matches_definition(lib, name):
    cfg = CONFIGS[name]
    dims = dims_of(lib, cfg, 1)
    say("w8 pack", name)
    buf = to_host(_w8_buffer(lib, cfg, dims))
    w = _w8_host(weight_key(cfg))
    want = packed_ref.w8_buffer(w["q_gate"], w["s_gate"], w["q_up"], w["s_up"], w["q_down"],
                                w["s_down"], w["qs_gate"], w["ss_gate"], w["qs_up"], w["ss_up"],
                                w["qs_down"], w["ss_down"])
    assert buf.size == want.size
    np.testing.assert_array_equal(buf, want)


@pytest.mark.gpu
@pytest.mark.parametrize("name,experts", [("W1", None), ("W2", None), ("C1", (0, 21, 63))])
def test_w8_quantize_matches_oracle(lib, name, experts):
    import torch
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, 1)
    dims = dims_of(lib, cfg, 1)
    buf = _empty((lib.w8_weights_size(dims),), torch.uint8)
    say("w8 quantize", name)
    lib.quantize_weights_w8(dims, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"],
                            dw["ws_up"], dw["ws_down"], buf)
    torch.cuda.synchronize()
    u = packed_ref.w8_unpack(to_host(buf), cfg.d, cfg.N, cfg.inter, cfg.I_s, experts)
    for e in (range(cfg.N) if experts is None else experts):
        for key, src, skey in (("q_gate", inp.w_gate, "s_gate"), ("q_up", inp.w_up, "s_up"),
                               ("q_down", inp.w_down, "s_down")):
            q, s = O.w8_quantize(src[e], "bf16")
            np.testing.assert_array_equal(u[key][e], q, err_msg=f"{key} expert {e}")
            np.testing.assert_array_equal(u[skey][e], s, err_msg=f"{skey} expert {e}")
    for key, src, skey in (("qs_gate", inp.ws_gate, "ss_gate"), ("qs_up", inp.ws_up, "ss_up"),
                           ("qs_down", inp.ws_down, "ss_down")):
        q, s = O.w8_quantize(src, "bf16")
        np.testing.assert_array_equal(u[key], q, err_msg=key)
        np.testing.assert_array_equal(u[skey], s, err_msg=skey)


@pytest.mark.gpu
@pytest.mark.parametrize("name,T", [("W1", 1), ("W1", 16), ("W1", 64), ("W1", 65), ("W1", 300),
                                    ("W2", 7), ("W2", 100), ("W2", 333)])
def test_w8_layer_small(lib, name, T):
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    buf = _w8_buffer(lib, cfg, dims_of(lib, cfg, T))
    say("w8 layer", name, T)
    out = _run(lib, cfg, T, dw, buf, logits_in=scores)
    ref = _oracle(inp, _w8_host(weight_key(cfg)), cfg, scores, None)
    np.testing.assert_array_equal(out["idx"], ref["idx"])
    assert (out["gc"] == T * cfg.kp).all()
    err = normwise_rel_err(values(out["y"]), ref["y"])
    assert err <= tolerance(cfg), err


@pytest.mark.gpu
@pytest.mark.parametrize("name,T", [("C1", 64), ("C1", 17), ("C2", 456), ("C2", 129),
                                    ("C2", 300), ("C3", 4096)])
def test_w8_layer_decode_sizes(lib, name, T):
    # (the prefill batch too: every routed expert then takes about eight 64-row
    # tiles on int8 codes, the last one partial.  129 and 300 tokens: the shared
    # segment's 64-row int8 tiles with a partial last row tile, beside routed
    # experts that stream or take 64-row tiles)
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    scores = S.make_scores(cfg, T=T)
    buf = _w8_buffer(lib, cfg, dims_of(lib, cfg, T))
    say("w8 layer (decode size)", name, T)
    out = _run(lib, cfg, T, dw, buf, logits_in=scores)
    np.testing.assert_array_equal(out["idx"], O.route(scores, cfg.M, cfg.kp)["idx"])
    tok = S.sample_tokens(T, 24)
    ref = _oracle(inp, _w8_host(weight_key(cfg)), cfg, scores, tok)
    err = normwise_rel_err(values(out["y"])[tok], ref["y"])
    assert err <= tolerance(cfg), err


@pytest.mark.gpu
def test_w8_layer_with_router_at_c1(lib):
    # the bench's call: router scores computed on the GPU from x and W_r
    from tests.test_gpu_parity import _score_error_bound
    cfg, T = C1, 64
    inp, dw = layer_inputs(cfg, T)
    buf = _w8_buffer(lib, cfg, dims_of(lib, cfg, T))
    say("w8 layer with router", cfg.name, T)
    out = _run(lib, cfg, T, dw, buf)
    tok = S.sample_tokens(T, 16)
    ref = _oracle(inp, _w8_host(weight_key(cfg)), cfg, None, tok)
    bound = _score_error_bound(inp, cfg)
    assert (np.abs(out["logits"] - ref["logits64"]) <= bound).all()
    np.testing.assert_array_equal(out["idx"], ref["idx"])
    err = normwise_rel_err(values(out["y"])[tok], ref["y"])
    assert err <= tolerance(cfg), err


@pytest.mark.gpu
@pytest.mark.parametrize("name,T", [("W2", 50)])
def test_w8_quantize_then_layer(lib, name, T):
    # bf16 weights quantised on the GPU, then the int8 layer; the oracle quantises
    # the same weights itself
    import torch
    cfg = CONFIGS[name]
    inp, dw = layer_inputs(cfg, T)
    dims = dims_of(lib, cfg, T)
    buf = _empty((lib.w8_weights_size(dims),), torch.uint8)
    lib.quantize_weights_w8(dims, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"],
                            dw["ws_up"], dw["ws_down"], buf)
    scores = S.make_scores(cfg, T=T)
    say("w8 quantize + layer", name, T)
    out = _run(lib, cfg, T, dw, buf, logits_in=scores)
    w = {}
    for key, skey, src in (("q_gate", "s_gate", inp.w_gate), ("q_up", "s_up", inp.w_up),
                           ("q_down", "s_down", inp.w_down), ("qs_gate", "ss_gate", inp.ws_gate),
                           ("qs_up", "ss_up", inp.ws_up), ("qs_down", "ss_down", inp.ws_down)):
        w[key], w[skey] = O.w8_quantize(src, "bf16")
    ref = _oracle(inp, w, cfg, scores, None)
    err = normwise_rel_err(values(out["y"]), ref["y"])
    assert err <= tolerance(cfg), err
